/*
 * ringag.h — C ABI of libringag.so: one tensor-parallel rank's share of the ring-decomposed
 * all-gather + GEMM (AG+GEMM) and of its mirror, GEMM + reduce-scatter (GEMM+RS), on one
 * AMD Instinct MI355X (gfx950).
 *
 * Pages the operations come from (cited by title and section):
 *   - TransformerEngine issue #1583 "curious about atomic_gemm_overlap_ag", C++ listing:
 *     a ring of tp-1 send/receive steps fills a gathered buffer chunk by chunk; one GEMM launch
 *     split into tp pieces along n waits on a per-chunk counter bumped after each receive; the
 *     output goes through a buffer of tp+1 chunks; the GEMM is "TN" (m = weight rows, n = gathered
 *     rows); communication runs on its own streams, forked from and joined to the main one.
 *   - nvFuser PR #3392 "Ring-based decomposition for Allgather+GEMM overlap ATen implementation",
 *     experiment: posting communication before compute gave near-complete overlap.
 *   - TransformerEngine PR #2443 "Comm+GEMM overlap API updated to support cuBlasMp backend",
 *     sequence diagram: AG+GEMM and GEMM+RS as the two phases of one context object with
 *     create/destroy; review comments: global k = local k * tp for the RS GEMM, argument-order
 *     mistakes between tp_rank and tp_size.
 *   - nvFuser PR #5742 "Reference implementation for Linear+Allreduce with overlapping",
 *     walkthrough: the chunked row-parallel linear equals the unchunked one; each output chunk is a
 *     sum over ranks.
 *
 * Simulated ring: the library runs one rank (self_rank) of a tp-rank ring on a single GPU.  The
 * other ranks' chunks are caller-provided device buffers; their "arrival" is a device-to-device
 * copy into the gathered buffer, in ring order, each followed by a bump of that chunk's ready
 * counter.  The copies run inside the GEMM launch itself (RAG_COPY_IN_GEMM, the default) or on a
 * library-owned side stream (RAG_COPY_KERNEL, RAG_COPY_SDMA).  A rank sends to rank+1 and receives from rank-1, so chunks
 * reach self_rank in the order s, s-1, s-2, ... (mod tp).
 *
 * Conventions for every entry point:
 *   - Tensor pointers are DEVICE pointers (memory from hipMalloc / torch on the context's device),
 *     owned by the caller, row-major, 16-byte aligned, and must stay valid until `stream` has
 *     passed the operation.  Host arrays of pointers (B_chunks, partials) are read during the call
 *     only.
 *   - Every call is stream-ordered on `stream` (0 = the null stream): it enqueues work and returns.
 *     Outputs are valid in `stream` order.  A side stream that carries copies starts after the
 *     work already in `stream` (event fork), and the call's last kernel on `stream` completes
 *     only after every copy of the call has completed (its workgroups wait for the copy counters
 *     or run the copies themselves; with RAG_COPY_ONLY on the side stream, `stream` waits for an
 *     event of the side stream instead).  So in `stream`
 *     order the inputs may be reused and the outputs are complete.
 *   - One operation in flight per context; a context is not thread-safe.  Consecutive calls on
 *     one context must be ordered: issue them on one stream, or make a later call's stream wait
 *     for the earlier call's (they share the context's counters).  Calls on different contexts
 *     are independent.
 *   - Every entry point returns RAG_OK (0) or a negative RAG_E* code and never throws.  Arguments
 *     are validated before any device work is enqueued; on failure nothing is enqueued and
 *     rag_last_error() describes the problem.
 *   - Integer order is always (tp, self_rank).
 */
#ifndef RINGAG_H
#define RINGAG_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__) || defined(__clang__)
#define RAG_API __attribute__((visibility("default")))
#else
#define RAG_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes. */
enum {
    RAG_OK = 0,
    RAG_EINVAL = -1,    /* bad argument; nothing was enqueued */
    RAG_EHIP = -2,      /* a HIP runtime call failed (message names it) */
    RAG_ETIMEOUT = -3,  /* a chunk's ready counter did not reach the call's epoch within the spin
                           limit; the tiles that waited were skipped (reported by rag_check) */
    RAG_ENOMEM = -4     /* a library-owned buffer could not be allocated */
};

/* Element types of the GEMM inputs, and of ag_gemm_ex's output D (bf16 unless ag_gemm_ex asks for
 * E4M3; every other entry point writes bf16). */
typedef enum {
    RAG_BF16 = 0,       /* bfloat16 */
    RAG_FP8_E4M3 = 1    /* OCP FP8 E4M3 (no infinities, max 448) with one fp32 scale per tensor */
} rag_dtype;

/* Flags for ag_gemm, gemm_rs and gemm_rs_ring (bitwise or). */
enum {
    RAG_STAGED_OUT = 1, /* AG+GEMM: write the output through a library-owned buffer of tp+1 chunks
                           in consumption order and copy it to D afterwards (the listing's output
                           staging); the default writes each chunk at its rank offset directly */
    RAG_NO_COPY = 2,    /* AG+GEMM: no arrivals; every chunk counts as ready and is read from its
                           slot of G as it is (GEMM-only timing; G must already hold the chunks) */
    RAG_COPY_ONLY = 4,  /* AG+GEMM: arrivals (copies + counter bumps) only, no GEMM */
    RAG_PER_CHUNK = 8,  /* AG+GEMM, split form: one GEMM launch per chunk in ring order on `stream`,
                           each waiting for its chunk's copy through a stream event instead of an
                           in-kernel counter (TransformerEngine PR #2443, sequence diagram: the
                           split overlap path; nvFuser PR #3392, experiment: one GEMM per received
                           chunk).  The copies always run on the side stream (the copy kernel, or
                           SDMA with RAG_COPY_SDMA); the per-tile trace is not recorded and the
                           withhold hook does not apply */
    RAG_RS_ARRIVE = 16  /* gemm_rs, gemm_rs_ring: the peers' data for this rank (gemm_rs: their
                           partials of the own chunk; gemm_rs_ring: the incoming running sums)
                           arrives during the call: the side stream copies it in ring order into a
                           library receive buffer, each copy releasing a counter, and a tile waits
                           for the counters of what its epilogue reads after its K loop (the
                           "atomic" reduce-scatter).  Needs the row stride equal to Mo.  With
                           RAG_COPY_IN_GEMM the GEMM+RS launch runs the copies itself (a waiting
                           tile copies until its counter is released, every workgroup copies a
                           share after each tile and the rest before it exits), except inside
                           rag_linear_allreduce, whose gather copies then run beside it: there,
                           and with RAG_COPY_KERNEL, the copy kernel on the side stream runs them;
                           with RAG_COPY_SDMA, SDMA */
};

/* Copy engines of the simulated arrival (RAG_OPT_COPY_ENGINE). */
enum {
    RAG_COPY_KERNEL = 0,   /* a copy kernel on the side stream, beside the GEMM.  Its waves need
                              room on every compute unit: with the automatic tile, a GEMM kernel
                              that leaves none gives way to one of the same tile size that does,
                              else 8 compute units are left out of the GEMM's grid */
    RAG_COPY_SDMA = 1,     /* SDMA engines on the side stream (hipMemcpyDeviceToDeviceNoCU, then
                              hipStreamWriteValue32 of the counter; RAG_OPT_SDMA_STREAMS spreads
                              the copies over up to three streams).  The runtime runs the
                              write-value as a small kernel on the compute units, so a GEMM whose
                              tiles wait for it leaves it room as for the copy kernel */
    RAG_COPY_IN_GEMM = 2,  /* the GEMM launch itself: workgroups whose chunk is not there yet copy
                              pieces of the peers' chunks (ring order) until it is released, and
                              help with the rest once out of tiles (in a launch of one persistent
                              round the own chunk's workgroups also copy one piece each before
                              their tile); no side stream is used (see
                              RAG_RS_ARRIVE for the GEMM+RS form).  With K-slab gating
                              (RAG_OPT_AG_GATE), every workgroup copies its share of slab pieces
                              instead, and a tile waits only for the slab it loads next */
    RAG_COPY_IN_GEMM_ASSIST = 3, /* AG+GEMM: as RAG_COPY_IN_GEMM, and a copy kernel on the side
                              stream takes pieces from the same queue beside the GEMM
                              (RAG_OPT_COMM_WGS workgroups): the chunks that only later rounds of
                              the GEMM need are copied while the first round computes, instead of
                              at the round boundary.  GEMM+RS calls treat it as RAG_COPY_IN_GEMM */
    RAG_COPY_IN_GEMM_SDMA = 4  /* AG+GEMM: as RAG_COPY_IN_GEMM for the chunks the first round of the
                              GEMM reads, and SDMA (as RAG_COPY_SDMA, over RAG_OPT_SDMA_STREAMS
                              streams) for the chunks only later rounds read: those are copied in
                              the background while the first round computes, on no compute unit.
                              The GEMM leaves room for the runtime's write-value kernel as with
                              RAG_COPY_SDMA.  One round: the same as RAG_COPY_IN_GEMM.  GEMM+RS
                              calls treat it as RAG_COPY_IN_GEMM */
};

/* Option keys for rag_set_option. */
enum {
    RAG_OPT_COPY_ENGINE = 1,    /* a RAG_COPY_* value (default RAG_COPY_IN_GEMM) */
    RAG_OPT_COMM_WGS = 2,       /* workgroups of the side-stream copy kernel (default 128,
                                   1..1024): the share of compute units that communication takes
                                   (gated rs_8k: 0.75 ms per call with 32, 0.45 with 128) */
    RAG_OPT_SPIN_LIMIT_US = 3,  /* how long a tile waits for its chunk before giving up
                                   (microseconds, default 2,000,000) */
    RAG_OPT_ARRIVAL_DELAY_US = 4, /* test hook: the kernel copy engines hold each counter bump back
                                   by this many microseconds after the chunk's copy (default 0,
                                   max 10^6) */
    RAG_OPT_WITHHOLD_MASK = 5,  /* test hook: bit j set = never bump the counter of the chunk at
                                   ring position j (1..tp-1); the waiting tiles then time out */
    RAG_OPT_TIMING = 6,         /* 1 = time every GEMM call (rag_kernel_times): a call that is one
                                   GEMM launch has the launch record its events itself (the
                                   kernel's duration); the split form, its launches together */
    RAG_OPT_TILE = 7,           /* GEMM tile configuration: 0 = automatic, else a RAG_TILE_* value */
    RAG_OPT_TRACE_BUF = 8,      /* diagnostics: device address of a buffer of 64-bit words that the
                                   next ag_gemm calls fill with wall-clock stamps (100 MHz): words
                                   0..tp-2 = release time of the chunk at ring position 1..tp-1,
                                   word tp-1 = completion of the own chunk's copy into G, word 32
                                   = start of the copies, then 5 words per GEMM tile in ring order
                                   from word 64 (start, after its wait, end, location = workgroup
                                   << 32 | XCC << 16 | SE << 8 | CU, core clock cycles from after
                                   the wait to the end); 0 = off (default) */
    RAG_OPT_TRACE_BYTES = 9,    /* diagnostics: size of that buffer; a call whose stamps would not
                                   fit records none */
    RAG_OPT_WGS_PER_CU = 10,    /* GEMM workgroups resident per compute unit: 0 = as many as fit
                                   (default), n = at most n (fewer, longer-lived workgroups take the
                                   ring's chunks in more rounds) */
    RAG_OPT_COPY_PRIORITY = 11, /* 1 (default) = copy-kernel waves issue at the highest wave
                                   priority, 0 = normal */
    RAG_OPT_GEMM_COPY_WGS = 12, /* RAG_COPY_IN_GEMM, AG+GEMM calls: how many of the GEMM's
                                   workgroups take part in the copies, spread evenly over the XCDs
                                   (0 = all, the default; GEMM+RS always uses all);
                                   fewer copy more slowly but draw less power at once */
    RAG_OPT_COMM_CUS = 13,      /* compute units given to communication: 0 (default) = the side
                                   stream's copy kernels may run anywhere; n (a multiple of 8,
                                   8 <= n <= CUs - 8) = the side stream is recreated with a
                                   compute-unit mask of n/8 units on every XCD, so copy kernels run
                                   only there (TransformerEngine issue #1583, C++ listing: the
                                   communication kernel gets its own number of SMs).  The GEMM's
                                   workgroups may share those units.  Such a stream is blocking with
                                   respect to the null stream: call from another stream, or the
                                   null stream serialises the copies with the GEMM */
    RAG_OPT_SDMA_STREAMS = 14,  /* RAG_COPY_SDMA: side streams the chunk copies are spread over
                                   (1..3, default 1), so that more than one copy engine works */
    RAG_OPT_AG_GATE = 15,       /* AG+GEMM with RAG_COPY_IN_GEMM: what a tile of a peer's chunk
                                   waits for.  RAG_GATE_CHUNK (default): the whole chunk (the
                                   listing's per-chunk counters).  RAG_GATE_SLAB: one K slab, where
                                   that applies (bf16 input, the 8-wave 2-stage tiles, G 128-byte
                                   aligned, no test hook set, not ag_gemm_noalloc; else by chunk):
                                   the peers' chunks are copied in pieces of 16 rows x 512 bytes of
                                   K, spread over every workgroup's K loop, and a tile waits for the
                                   pieces of the 4 K stages it loads next, so every tile starts at
                                   once.  The library's own addition: finer-grained gating of the
                                   same arrival */
    RAG_OPT_SLAB_HELP_US = 16   /* K-slab gating: how long a tile waits for a slab before its
                                   workgroup copies the slab's missing pieces itself (0..1e7 us,
                                   default 20; 0 = at once, a test hook for that path) */
};

/* Values of RAG_OPT_AG_GATE. */
enum { RAG_GATE_CHUNK = 0, RAG_GATE_SLAB = 1 };

/* Tile configurations (rows of D x columns of D per workgroup; 4 waves unless stated). */
enum { RAG_TILE_AUTO = 0, RAG_TILE_128x128 = 1, RAG_TILE_256x128 = 2,
       RAG_TILE_256x256 = 3 /* 4 waves of 128x128, 2 LDS stages of 128-byte rows */,
       RAG_TILE_256x256_8W = 4 /* 8 waves of 128x64, 2 LDS stages of 128-byte rows */,
       RAG_TILE_256x256_8W_S4 = 5 /* 8 waves of 128x64, 4 LDS stages of 64-byte rows */,
       RAG_TILE_256x192_8W = 6 /* 8 waves of 64x96, 2 LDS stages of 128-byte rows */ };

typedef struct rag_ctx rag_ctx;     /* opaque; owned by the library */

#define RAG_MAX_TP 16

/* Create a context on `device` for rings of up to max_tp ranks (1..RAG_MAX_TP).  Allocates the
 * side stream, events, per-chunk ready counters, an error word and the epoch (all cached for the
 * context's life; no per-call allocation).  flags: reserved, pass 0.  On success *out receives the
 * context.  TransformerEngine PR #2443, sequence diagram: context creation at initialisation. */
RAG_API int rag_create(rag_ctx** out, int device, int max_tp, int flags);

/* Destroy a context: waits for its side stream, then destroys its streams and events and frees
 * its counters and cached buffers.  Safe on NULL; always returns RAG_OK.  TransformerEngine PR
 * #2443, sequence diagram, cleanup phase: the overlap object's destructor destroys the context
 * (nvte_comm_gemm_ctx_destroy) or, on the other backend, its streams and events. */
RAG_API int rag_destroy(rag_ctx* ctx);

/* Set an option (RAG_OPT_*).  Takes effect from the next call.  The library's own addition (the
 * pages configure their overlap objects through constructor arguments): engine, tile and test-hook
 * settings that the tests and the benchmark change between calls.  RAG_EINVAL for an unknown key
 * or a value out of range (nothing changes then). */
RAG_API int rag_set_option(rag_ctx* ctx, int key, long long value);

/*
 * AG+GEMM for rank self_rank of a tp-rank ring:
 *     G = [B_0; B_1; ...; B_{tp-1}]          (rank-ordered all-gather, chunk r at row r*nc)
 *     D = G * A^T                            (bf16 out, fp32 accumulation)
 * TransformerEngine issue #1583, C++ listing (ring steps, per-chunk counters, split GEMM, TN
 * layout, N+1-chunk output staging); nvFuser PR #3392 (ring decomposition; communication posted
 * before compute).
 *
 *   A         weight shard [M, K], dt
 *   M, K      M >= 1; K >= 1 and a multiple of 64 (bf16) or 128 (fp8)
 *   B_chunks  HOST array of tp device pointers, B_chunks[r] = rank r's chunk [nc, K], dt.  Entry
 *             self_rank is this rank's own chunk (read directly, never waited for); the others
 *             stand for the peers' chunks and are copied into G as they "arrive".
 *   nc        rows per chunk (>= 1); N = tp * nc
 *   tp, self_rank  1 <= tp <= max_tp of the context, 0 <= self_rank < tp
 *   G         [N, K] dt, receives the gathered input (chunk r at rows [r*nc, (r+1)*nc)); NULL = use
 *             a library-owned gather buffer (then the gathered input is not returned)
 *   D         [N, M] bf16 output; chunk r's rows are B_r * A^T whatever self_rank is
 *   dt        RAG_BF16 or RAG_FP8_E4M3
 *   scale_A, scale_B  device fp32 scalars (dequantisation factors: value = code * scale); required
 *             for fp8, must be NULL for bf16
 *   flags     RAG_STAGED_OUT | RAG_NO_COPY | RAG_COPY_ONLY (NO_COPY and COPY_ONLY are exclusive)
 *   stream    caller's stream
 * Errors: RAG_EINVAL (bad sizes/pointers/flags, any operand of 2 GiB or more, G or D overlapping
 * an input), RAG_EHIP, RAG_ENOMEM.  A chunk that never arrives is reported by rag_check.
 */
RAG_API int ag_gemm(rag_ctx* ctx,
            const void* A, int M, int K,
            const void* const* B_chunks, int nc,
            int tp, int self_rank,
            void* G, void* D,
            rag_dtype dt, const float* scale_A, const float* scale_B,
            int flags, void* stream);

/*
 * ag_gemm with the output and save options of the listing's call (TransformerEngine issue #1583,
 * C++ listing: the output buffer carries D's amax and scale, and B_copy stores the rank's input
 * chunk for the backward pass).  Arguments as for ag_gemm, plus:
 *   d_dt      RAG_BF16 (D as in ag_gemm) or RAG_FP8_E4M3: D is [tp*nc, M] E4M3 codes,
 *             code = E4M3(v * scale_D[0]) with v the GEMM result (for fp8 inputs already
 *             multiplied by scale_A * scale_B), saturated to +-448, round to nearest even
 *   scale_D   device fp32 scalar; required for fp8 output, NULL otherwise
 *   amax_D    device fp32 scalar or NULL (fp8 output only): max |v| over D is max-reduced into
 *             it (the caller sets its starting value, e.g. 0)
 *   B_copy    device buffer [nc, K] in the input dtype, or NULL: receives this rank's chunk,
 *             copied by the same engine as the arrivals (RAG_NO_COPY skips it with them)
 * Errors: as ag_gemm.
 */
RAG_API int ag_gemm_ex(rag_ctx* ctx,
            const void* A, int M, int K,
            const void* const* B_chunks, int nc,
            int tp, int self_rank,
            void* G, void* D,
            rag_dtype dt, const float* scale_A, const float* scale_B,
            rag_dtype d_dt, const float* scale_D, float* amax_D, void* B_copy,
            int flags, void* stream);

/*
 * ag_gemm for callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): the call's ready counters, piece counts and
 * error word live in a fixed array of the library's code object, RAG_SCRATCH_BYTES per device
 * (set up and cleared when the first context on the device is created, kept until the process
 * ends), instead of the context's own allocation.  The call allocates nothing.
 *   Arguments as for ag_gemm, except: G is required (not NULL); flags may hold only RAG_NO_COPY or
 *   RAG_COPY_ONLY (RAG_STAGED_OUT and RAG_PER_CHUNK use a buffer and events that the library
 *   allocates on first use); tp <= RAG_MAX_TP, the most the array holds words for.
 *   Every call on a device shares that device's array, with every context there: calls that
 *   overlap on one device race (their counters and piece counts collide), so they must be ordered
 *   like calls on one context.  The array keeps the last call's contents; the counters are compared
 *   with a per-device epoch that rises with every call, and each launch clears the piece counts
 *   the next call uses, so nothing needs clearing between calls.  A wait that times out is
 *   reported by rag_check on any context of the device.
 * Errors: RAG_EINVAL (as ag_gemm, plus a NULL G, a forbidden flag, tp > RAG_MAX_TP), RAG_EHIP.
 */
#define RAG_SCRATCH_BYTES 22016
RAG_API int ag_gemm_noalloc(rag_ctx* ctx,
            const void* A, int M, int K,
            const void* const* B_chunks, int nc,
            int tp, int self_rank,
            void* G, void* D,
            rag_dtype dt, const float* scale_A, const float* scale_B,
            int flags, void* stream);

/*
 * GEMM + reduce-scatter (row-parallel linear) for rank self_rank of a tp-rank ring:
 *     P     = X * W^T over all T rows            (this rank's partial of the full output, fp32)
 *     D     = sum over ranks p of P_p[rows of chunk self_rank]   (bf16 out)
 *     send[c] = P[rows of chunk c]  for c != self_rank            (fp32, the outgoing chunks)
 * where P_p for p != self_rank are the peers' partials given in `partials`.
 * TransformerEngine PR #2443 (sequence diagram: split GEMM then reduce-scatter; review: the RS
 * GEMM's contraction dimension is the local shard of a global k); nvFuser PR #5742 (walkthrough:
 * each output chunk is summed over ranks).
 *
 *   X         [T, Kl] bf16 activation shard; T = tp * nc
 *   W         [Mo, Kl] bf16 weight shard
 *   Kl        >= 1, multiple of 64;  Mo >= 4, multiple of 4, <= 2^20
 *   partials  HOST array of tp device pointers to fp32 [T, Mo] partials with row stride ldp
 *             (elements, Mo <= ldp <= 2^20, 4-byte aligned); only rows of chunk self_rank are
 *             read (memory from the chunk's first element to its last must be readable); entry
 *             self_rank ignored
 *   send      [tp, nc, Mo] fp32 outgoing chunks (slot self_rank untouched); NULL = not stored
 *   D         [nc, Mo] bf16, this rank's reduced chunk
 *   flags     0 or RAG_RS_ARRIVE
 * Row chunks are computed in the order c_j = (self_rank + 1 + j) mod tp, the own chunk last.
 * Errors: RAG_EINVAL, RAG_EHIP; with RAG_RS_ARRIVE, rag_check reports RAG_ETIMEOUT for a copy
 * that never completes.
 */
RAG_API int gemm_rs(rag_ctx* ctx,
            const void* X, int T, int Kl,
            const void* W, int Mo,
            const float* const* partials, long long ldp,
            int tp, int self_rank,
            float* send, void* D,
            int flags, void* stream);

/* Synchronise the context's device (hipDeviceSynchronize) and report whether any wait of a
 * counter-gated tile timed out since the last check: RAG_ETIMEOUT (the error word is then cleared
 * and the message names the call's epoch), or RAG_OK.  The library's own addition: the pages'
 * counter waits have no time limit; here a wait is bounded (RAG_OPT_SPIN_LIMIT_US) so that a
 * chunk that never arrives ends as an error instead of a hang.  Errors: RAG_EINVAL (NULL ctx),
 * RAG_EHIP. */
RAG_API int rag_check(rag_ctx* ctx);

/* GEMM kernel durations (milliseconds) recorded since the last call to this function while
 * RAG_OPT_TIMING was on; synchronises those events.  Writes up to max_n values to out and returns
 * how many were recorded (>= 0), or a negative RAG_E* code.  The library's own addition, for
 * measurement: the pages time their kernels with a profiler (nvFuser PR #5742, nsys trace), which
 * this gives without one. */
RAG_API int rag_kernel_times(rag_ctx* ctx, float* out, int max_n);

/* Name of the GPU kernel entry point a chunked ag_gemm call (bf16 output) would launch for these
 * sizes (nc rows per chunk, M output columns, tp chunks) with the context's current options (e.g.
 * "rag_ag_bf16_t256x256w8"), written NUL-terminated into buf (len bytes).  Diagnostics, the
 * library's own addition: lets a profile be matched to the kernel a measurement ran. */
RAG_API int rag_ag_kernel_name(rag_ctx* ctx, int nc, int M, int tp, rag_dtype dt, char* buf,
                               int len);

/*
 * One rank's step of a ring-accumulate reduce-scatter (the running sums go to rank self_rank+1):
 *     P       = X * W^T over all T rows
 *     send[c] = incoming[c] + P[rows of chunk c]   for c != self_rank    (fp32, passed on)
 *     D       = incoming[self_rank] + P[rows of chunk self_rank]        (bf16, the reduced chunk)
 * where incoming[c] is the running sum of chunk c that arrives from rank self_rank-1, and the
 * chain of chunk (self_rank-1) mod tp starts here (no incoming: send = P's rows).  Chunks are
 * computed in the ring order c_k = (self_rank - 1 - k) mod tp, the own chunk last.
 * TransformerEngine PR #2443 (sequence diagram: split GEMM then reduce-scatter);
 * nvFuser PR #5742 (walkthrough: each output chunk is summed over ranks).
 *
 *   X, W, Kl, Mo, send, D as for gemm_rs (send NULL = the passed-on sums are not stored)
 *   incoming  HOST array of tp device pointers to fp32 [nc, Mo] running sums with row stride ldi
 *             (elements, Mo <= ldi <= 2^20, 4-byte aligned); entry (self_rank - 1) mod tp ignored
 *   flags     0 or RAG_RS_ARRIVE
 * Errors: RAG_EINVAL, RAG_EHIP (RAG_ETIMEOUT through rag_check as for gemm_rs).
 */
RAG_API int gemm_rs_ring(rag_ctx* ctx,
            const void* X, int T, int Kl,
            const void* W, int Mo,
            const float* const* incoming, long long ldi,
            int tp, int self_rank,
            float* send, void* D,
            int flags, void* stream);

/*
 * One rank's share of a row-parallel linear whose output is all-reduced, as a reduce-scatter
 * followed by an all-gather of the reduced chunks (nvFuser PR #5742, walkthrough and sequence
 * diagram: per-chunk matmul, then that chunk's all-reduce; TransformerEngine PR #2443, sequence
 * diagram: reduce-scatter of the split GEMM):
 *     Y[rows of chunk self_rank] = sum over ranks of P_p[rows of chunk self_rank]  (gemm_rs)
 *     Y[rows of chunk c]         = reduced[c]  for c != self_rank (the owners' reduced chunks,
 *                                  all-gathered: copied in ring order, self_rank-1 first,
 *                                  by the GEMM+RS launch's own workgroups after their tiles
 *                                  with RAG_COPY_IN_GEMM and no RAG_RS_ARRIVE, else by the
 *                                  side stream while the GEMM runs)
 *     send                       as for gemm_rs
 *
 *   X, W, Kl, partials, ldp, send, flags as for gemm_rs
 *   Mo        >= 8, multiple of 8
 *   reduced   HOST array of tp device pointers to bf16 [nc, Mo] reduced chunks (contiguous);
 *             entry self_rank ignored
 *   Y         [T, Mo] bf16 output, T = tp * nc
 * Engines of the all-gather's copies: with RAG_COPY_IN_GEMM and no RAG_RS_ARRIVE, the GEMM+RS
 * launch's own workgroups (after their tiles); with RAG_COPY_IN_GEMM and RAG_RS_ARRIVE, and with
 * RAG_COPY_KERNEL, the copy kernel on the side stream; with RAG_COPY_SDMA, SDMA on the side
 * stream.  Side-stream copies are joined back into `stream` before the call's later work.
 * Errors: RAG_EINVAL, RAG_EHIP.
 */
RAG_API int linear_allreduce(rag_ctx* ctx,
            const void* X, int T, int Kl,
            const void* W, int Mo,
            const float* const* partials, long long ldp,
            const void* const* reduced,
            int tp, int self_rank,
            float* send, void* Y,
            int flags, void* stream);

/* Name of the GPU kernel entry point gemm_rs would launch for these sizes (nc rows per chunk, Mo
 * output columns, tp chunks) with the context's current options (e.g. "rag_rs_t256x256w8").
 * Diagnostics, the library's own addition, like rag_ag_kernel_name. */
RAG_API int rag_rs_kernel_name(rag_ctx* ctx, int nc, int Mo, int tp, char* buf, int len);

/* Text for the last non-zero return on the calling thread ("" if none): names the entry point,
 * the offending argument and its value, or the HIP call and its error string.  TransformerEngine
 * PR #2443, review comments: an error message should say what was chosen and what it requires
 * instead of only that something failed. */
RAG_API const char* rag_last_error(void);

/* Library version, major * 10000 + minor * 100 + patch.  The library's own addition. */
RAG_API int rag_version(void);

#ifdef __cplusplus
}
#endif

#endif /* RINGAG_H */
