// Internal interface shared by the host runtime (runtime.cpp, launch.cpp) and the device code
// (device_kernels.hip): kernel argument structs, tile geometry and the tile-to-XCD mapping.
// Nothing here is part of the public ABI.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

#ifndef __HIPCC__
#define RAG_HD
#else
#define RAG_HD __host__ __device__
#endif

namespace ringag {

constexpr int kMaxTp = 16;

// Device counters live kWordStride ints apart (256 bytes), one per cache line: the GEMM's tiles
// poll the ready counters continuously, and an atomic on a line that is being polled queues
// behind the polls.
constexpr int kWordStride = 64;

// The copies of one call's simulated arrival, as a queue of pieces (copy kernel on the side
// stream, or the GEMM's own workgroups while their chunk is not there yet).  Copies
// 0..n_peer-1 are the peers' chunks in ring order; each releases ctr[ctr_index[c]] = epoch once
// all its pieces are copied.  Copy n_peer, when n > n_peer, is the own chunk into its slot of G
// (ctr_index -1 unless something waits for it).  Grab counts hand out the pieces of three queues
// in order: queue 0 (grab[0]) = the first n_peer - late peers, queue 2 (grab[2 kWordStride]) = the
// last `late` peers (chunks that only later rounds of the GEMM need, which a copy kernel beside it
// takes in the background), queue 1 (grab[kWordStride]) = the own chunk's copies;
// done[c * kWordStride] counts the copied pieces of copy c.  The counts come in two sets used by alternate calls; a
// launch zeroes the other set (clear_next, 2 * kArrSlots counts) for the next call.
constexpr int kArrSlots = kMaxTp + 1;   // copies per call at most (tp - 1 peers + the own chunk)

// Ints in one set of a call's device words for rings of up to kMaxTp ranks, kWordStride ints
// apart: ready counters [kMaxTp] | copy-complete counter | piece counts [2 sets][grab, done]
// [kArrSlots] | error word.  A context allocates this layout for its max_tp; the library's fixed
// scratch array (device_kernels.hip) holds it for kMaxTp (22 KiB).
constexpr int kScratchWords = (kMaxTp + 1 + 4 * kArrSlots + 1) * kWordStride;

struct CopyPlan {
  const void* src[kArrSlots];
  void* dst[kArrSlots];
  int ctr_index[kArrSlots];      // counter released when copy c is complete, or -1
  int pos[kArrSlots];            // ring position of copy c (withhold hook); 0 = the own chunk
  int n_peer, n;
  int late;                      // the last `late` of the n_peer peer copies form queue 2
  int late_external;             // 1 = SDMA copies queue 2 (and releases its counters): no
                                 // kernel takes its pieces
  unsigned long long bytes;      // bytes per copy, multiple of 16
  unsigned pieces;               // pieces per copy: ceil(bytes / piece_bytes)
  unsigned piece_bytes;          // multiple of 16
  unsigned* grab;
  unsigned* done;
  unsigned* clear_next;
  long long delay_ticks;         // test hook: hold each release back this long
  unsigned withhold_mask;        // test hook: bit pos (>= 1) set = never release that chunk
  unsigned long long* trace;     // optional: [c] = completion time of copy c, [kTraceStart] = start
};

// K-slab gating of the in-GEMM copies (AG+GEMM, bf16, 8-wave tiles with 2 stages of 128 bytes).
// The peers' chunks are cut into pieces of kSlabRows rows by kSlabRowBytes bytes of K (one group
// of kSlabStages K stages), numbered group by group: piece (g, c, rb) = rows [rb * kSlabRows, +
// kSlabRows) of group g of copy c, index (g * n_peer + c) * ppc + rb.  Piece i belongs to
// workgroup (i / q) % grid, which copies it in its slot i / (q * grid): slots 0 .. pre-1 before
// its first tile, later ones one per group of K stages inside its K loops, and whatever is left
// after its last tile.  flags[(c * groups + g) * ppc + rb] holds the epoch of the last call that
// copied that piece; a tile of chunk c waits for all ppc flags of group g before loading it, and
// copies the missing pieces itself once it has waited help_ticks.
constexpr int kSlabRowBytes = 512;
constexpr int kSlabRows = 16;       // 16 rows x 512 bytes = 8 KiB: one 16-byte vector per thread
constexpr int kSlabThreads = 512;
constexpr int kSlabStages = 4;      // K stages of 128 bytes per group
constexpr int kSlabMaxQ = 2;        // pieces per slot at most

struct SlabPlan {
  int on;                        // 1 = the peers' chunks are copied and waited for by K slab
  int groups;                    // groups of K per row: ceil(K bytes / kSlabRowBytes)
  int ppc;                       // pieces per chunk and group: ceil(nc / kSlabRows)
  int q;                         // pieces per slot (1 .. kSlabMaxQ)
  int pre;                       // slots copied before the first tile
  int total;                     // pieces of the call: groups * n_peer * ppc
  long long help_ticks;          // wall-clock ticks a tile waits before copying missing pieces
  int* flags;                    // [n_peer][groups][ppc] epochs
};

// Arguments of the counter-gated AG+GEMM kernel.  Chunk positions j = 0..tp-1 are the ring order
// at this rank (position 0 = own chunk).
struct AgArgs {
  const void* chunk[kMaxTp];     // by position: where the kernel reads that chunk's rows
  void* out[kMaxTp];             // by position: where that chunk's [nc, M] bf16 output rows go
  int ctr_index[kMaxTp];         // by position: counter to wait for, -1 = ready from the start
  int join_index;                // counter marking the copy into the own slot of G done, or -1:
                                 // every workgroup waits for it before it exits
  const void* A;                 // weight [M, K]
  int M, K, nc, tp;
  int* ctr;                      // per-chunk ready counters (kWordStride apart)
  int epoch;                     // value meaning "ready" for this call
  int* err;                      // error word: set to the epoch when a wait times out
  long long spin_limit;          // wall-clock ticks a tile waits before giving up
  const float* scale_A;          // fp8: dequantisation factors (device scalars)
  const float* scale_B;
  int tiles_i, tiles_j;          // tile grid of one chunk
  unsigned long long* trace;     // optional per-tile stamps (kTraceTileWords per tile), or null
  int out_fp8;                   // 1 = D is E4M3: code = E4M3(acc * scale * scale_D[0])
  const float* scale_D;          // fp8 output: quantisation factor (device scalar)
  float* amax_D;                 // fp8 output, optional: max |acc * scale| is max-reduced into it
  int copies;                    // 1 = this kernel also runs the copies of `cp`
  int copy_stride;               // workgroups w with (w / 8) % copy_stride == 0 copy
  int compute;                   // 0 = copies only, no tiles
  CopyPlan cp;
  SlabPlan slab;                 // slab.on: the peers' copies (cp 0 .. n_peer-1) go by K slab
};

// Arguments of the GEMM+RS kernel.  Row-chunk positions j = 0..tp-1 in visiting order; the last
// one is this rank's own chunk.  Two forms: the one-shot reduce-scatter (ring = 0: tiles of other
// chunks store their fp32 accumulators to send, the own chunk's tiles add every peer's partial of
// the own chunk) and one ring-accumulate step (ring = 1: the tiles of chunk c add the running sum
// of chunk c that arrives from the previous rank, then store to send, or to D for the own chunk).
struct RsArgs {
  const void* X;                 // [T, Kl] bf16
  const void* W;                 // [Mo, Kl] bf16
  int chunk_of[kMaxTp];          // by position: row chunk index c
  const float* partial[kMaxTp];  // ring = 0: by rank p, p's partial rows of the own chunk;
                                 // ring = 1: by chunk c, the incoming running sum (or null);
                                 // [nc, Mo] fp32 with row stride ldp
  long long ldp;
  int ring;
  float* send;                   // [tp, nc, Mo] fp32 or null
  void* D;                       // [nc, Mo] bf16
  int T, Kl, Mo, nc, tp, self_rank;
  int tiles_i, tiles_j;
  int gated;                     // 1 = the data of partial[] arrives during the call: a tile waits
                                 // for the counters of what its epilogue reads (ctr, by rank for
                                 // ring = 0, by chunk for ring = 1)
  int* ctr;
  int epoch;
  int* err;
  long long spin_limit;
  int copies;                    // 1 = this kernel also runs the copies of `cp` (gated only): a
                                 // tile copies until the counter it waits for is released, and
                                 // every workgroup copies up to copy_quota pieces after each tile
  int copy_quota;
  CopyPlan cp;
};

// Arguments of the arrival (producer) kernel on the side stream: runs the whole piece queue.
struct ArrivalArgs {
  CopyPlan cp;
  int* ctr;
  int epoch;
  int raise_priority;            // 1 = run the copy waves at the highest issue priority
  int late_only;                 // 1 = only queues 2 and 1 (beside a GEMM whose own workgroups
                                 // copy queue 0)
};

// Trace layout (64-bit words, wall clock at 100 MHz): words [0, kTraceHeader) belong to the
// copies (completion time of copy c at [c], start of the first copying launch at [kTraceStart]);
// tile t of the GEMM (ring-ordered index) owns words kTraceHeader + 5 t .. + 4: start (before its
// wait), after the wait, end (after its stores), (workgroup << 32) | (XCC << 16) | (SE << 8) | CU,
// and the core clock cycles (s_memtime) from after the wait to the end, so that cycles / wall
// time gives the clock the tile ran at.
constexpr int kTraceHeader = 64;
constexpr int kTraceStart = 32;
constexpr int kTraceTileWords = 5;

enum TileCfg {
  kTile128x128 = 1, kTile256x128 = 2, kTile256x256 = 3, kTile256x256w8 = 4, kTile256x256w8s4 = 5,
  kTile256x192w8 = 6
};
constexpr int kNumTiles = 7;   // tile ids 1 .. kNumTiles - 1

struct KernelInfo {
  int threads;
  int lds_bytes;
  int vgprs_per_wave;   // arch + acc registers, as reported by the runtime
  int max_blocks_per_cu;
};

// Kernel loading and launching (launch.cpp).  load_kernels loads the embedded code object on
// `device` once per process (kept until the process ends, so nothing of the library runs at exit);
// the launchers enqueue on `stream` (the current device must be `device`) and return the
// hipError_t of the launch; given ev_start / ev_stop, the launch itself records them around the
// kernel.
hipError_t load_kernels(int device);
// The device address of the fixed scratch array in the code object loaded on `device` (looked up
// once, when load_kernels loads the module there, and cleared then); null before that.
int* device_scratch(int device);
hipError_t launch_ag_gemm(int device, const AgArgs& a, int tile, bool fp8, int grid,
                          hipStream_t stream, hipEvent_t ev_start = nullptr,
                          hipEvent_t ev_stop = nullptr);
hipError_t launch_gemm_rs(int device, const RsArgs& a, int tile, int grid, hipStream_t stream,
                          hipEvent_t ev_start = nullptr, hipEvent_t ev_stop = nullptr);
hipError_t launch_arrival(int device, const ArrivalArgs& a, int grid, hipStream_t stream);

// Entry-point names (launch.cpp); "" when there is none (slab: the K-slab-gated form).
const char* ag_kernel_name(int tile, bool fp8, bool out8 = false, bool slab = false);
// Whether a tile configuration has K-slab-gated kernels.
bool ag_slab_tile(int tile);
const char* rs_kernel_name(int tile);

// Occupancy / resource facts for a kernel variant (cached by the caller).
hipError_t ag_kernel_info(int device, int tile, bool fp8, bool out8, KernelInfo* info);
hipError_t rs_kernel_info(int device, int tile, KernelInfo* info);
hipError_t arrival_kernel_info(int device, KernelInfo* info);

constexpr int kArrivalThreads = 256;   // block size of the arrival kernel

// Threads per workgroup of a tile configuration (4 waves, or 8 for the 8-wave tiles).
inline int tile_threads(int tile) {
  return (tile == kTile256x256w8 || tile == kTile256x256w8s4 || tile == kTile256x192w8) ? 512
                                                                                      : 256;
}

// Tile sizes of a configuration.
inline void tile_dims(int tile, int* bi, int* bj) {
  switch (tile) {
    case kTile256x256:
    case kTile256x256w8:
    case kTile256x256w8s4: *bi = 256; *bj = 256; break;
    case kTile256x192w8: *bi = 256; *bj = 192; break;
    case kTile256x128: *bi = 256; *bj = 128; break;
    default: *bi = 128; *bj = 128; break;
  }
}

}  // namespace ringag
