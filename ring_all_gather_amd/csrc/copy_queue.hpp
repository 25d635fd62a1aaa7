// The piece queue of a call's copies (the simulated arrival of the peers' chunks), run by whole
// workgroups: those of the arrival kernel on the side stream, or the GEMM's own workgroups while
// the chunk of their next tile is not there yet.
//
// TransformerEngine issue #1583, C++ listing: each ring step copies one chunk into the gathered
// buffer and then bumps that chunk's counter.  Here a chunk is cut into pieces; workgroups take
// pieces in ring order with an atomic, copy them, and add them to the chunk's done count.  The
// add that completes the count stores the chunk's counter.  Whoever takes a piece copies it
// without waiting on anything, so every chunk's count completes even when not all workgroups are
// resident.
//
// Visibility of the copied bytes: the pieces are stored with the agent-scope write-through policy
// (kCopyStorePolicy), every wave waits until its stores are complete before the workgroup's
// barrier, and only then does thread 0 add to the done count, an agent-scope atomic.  A store of
// that policy is visible device-wide once it is complete (it is how the memory model's own
// agent-scope atomic stores are built), so the count and the counter need no release: a release
// would add an L2 write-back of the copying XCD, which covers only lines that were not written
// through, and these copies leave none.  That write-back took about 2.3 us per piece whether or
// not there was anything to write, against ~4 us to copy a 128 KiB piece (copies-only ag_qkv 49
// -> 38 us, chunked 391 -> 359 us without it).  The consumer still takes an acquire fence after
// it sees the counter (wait_ready), which drops any stale line of the slot from its XCD's L2.
#pragma once

#include <hip/hip_runtime.h>

#include "kernels.hpp"

namespace ringag {

typedef int v4i __attribute__((ext_vector_type(4)));

// Wait until *ctr == epoch.  Returns false when the limit passed or another tile of this call
// already gave up (then *err == epoch).  The loop polls with relaxed agent-scope loads, which
// read the counter coherently without touching the caches; a single acquire fence after the
// value is seen orders the tile's loads of the chunk after the producer's counter store.  (An
// acquire load in the loop would invalidate this CU's cache lines on every poll, slowing the
// tiles and the copies that share the XCD.)
__device__ inline bool wait_ready(int* ctr, int epoch, int* err, long long limit) {
  bool ok = __hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == epoch;
  if (!ok) {
    const unsigned long long t0 = wall_clock64();
    while (true) {
      __builtin_amdgcn_s_sleep(8);
      if (__hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == epoch) {
        ok = true;
        break;
      }
      if (__hip_atomic_load(err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == epoch) break;
      if ((long long)(wall_clock64() - t0) > limit) {
        __hip_atomic_store(err, epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
    }
  }
  if (ok) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  return ok;
}

// Cache policy of the copies' stores: sc1, agent scope.  The data is written through the copying
// XCD's L2 to the point where every XCD sees it, instead of staying dirty in that L2 (ag_4k:
// copies-only launch 21.1 -> 18.0 us, chunked call 125.0 -> 120.6 us, when each piece still ended
// with a release that wrote the L2 back).
constexpr int kCopyStorePolicy = 16;

// Copy piece k of copy c with the NT threads of the workgroup (16-byte vectors, U in flight per
// thread).
template <int NT, int U, bool PIPE>
__device__ __forceinline__ void copy_piece(const CopyPlan& p, unsigned c, unsigned k) {
  const unsigned long long beg = (unsigned long long)k * p.piece_bytes;
  const unsigned long long len = min((unsigned long long)p.piece_bytes, p.bytes - beg);
  const v4i* s = (const v4i*)((const char*)p.src[c] + beg);
  const unsigned nvec = (unsigned)(len / 16);
  const __amdgpu_buffer_rsrc_t d = __builtin_amdgcn_make_buffer_rsrc(
      (char*)p.dst[c] + beg, 0, (int)(nvec * 16), 0x00020000);
  // PIPE: batches of U vectors per thread that every thread copies in full, software-pipelined:
  // the next batch's loads go out before this batch's stores, so the wait for a batch's loads
  // (vmcnt counts loads and stores in order) leaves the previous batch's stores and the next
  // batch's loads in flight (ag_4k copies-only launch 18.0 -> 17.4 us, ag_qkv 61.8 -> 57.1 us).
  // The trip count is uniform, so the compiler can count them.  It holds two batches in
  // registers, so the GEMM+RS kernel (which copies while its accumulators are live) and the
  // arrival kernel (whose waves must fit beside a GEMM's) use the plain loop: load a batch,
  // store it.
  unsigned i;
  if constexpr (PIPE) {
    const unsigned nb = nvec / (U * NT);
    const unsigned t0 = threadIdx.x;
    auto ld = [&](v4i(&r)[U], unsigned q) {
#pragma unroll
      for (int u = 0; u < U; ++u) r[u] = s[t0 + (q * U + u) * NT];
    };
    auto st = [&](const v4i(&r)[U], unsigned q) {
#pragma unroll
      for (int u = 0; u < U; ++u)
        __builtin_amdgcn_raw_buffer_store_b128(r[u], d, (int)((t0 + (q * U + u) * NT) * 16), 0,
                                               kCopyStorePolicy);
    };
    if (nb > 0) {
      // two register sets used in turn (no moves between them, which would wait for every load)
      v4i v[U], w[U];
      ld(v, 0);
      unsigned b = 1;
      for (; b + 1 < nb; b += 2) {
        ld(w, b);
        st(v, b - 1);
        ld(v, b + 1);
        st(w, b);
      }
      if (b < nb) {
        ld(w, b);
        st(v, b - 1);
        st(w, b);
      } else {
        st(v, b - 1);
      }
    }
    i = t0 + nb * U * NT;
  } else {
    i = threadIdx.x;
    for (; i + (U - 1) * NT < nvec; i += U * NT) {
      v4i v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) v[u] = s[i + u * NT];
#pragma unroll
      for (int u = 0; u < U; ++u)
        __builtin_amdgcn_raw_buffer_store_b128(v[u], d, (int)((i + u * NT) * 16), 0,
                                               kCopyStorePolicy);
    }
  }
  for (; i < nvec; i += NT)
    __builtin_amdgcn_raw_buffer_store_b128(s[i], d, (int)(i * 16), 0, kCopyStorePolicy);
}

// Thread 0, after the stores of `count` pieces of copy c by every wave of the workgroup are
// complete: add them to the copy's done count; the add that completes it stores the copy's
// counter (see the head of this file for why both are relaxed).
__device__ inline void pieces_done(const CopyPlan& p, int* ctr, int epoch, unsigned c,
                                   unsigned count) {
  const unsigned old = __hip_atomic_fetch_add(p.done + c * kWordStride, count, __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_AGENT);
  if (old + count != p.pieces) return;
  if (p.delay_ticks > 0) {
    const unsigned long long t0 = wall_clock64();
    while ((long long)(wall_clock64() - t0) < p.delay_ticks) __builtin_amdgcn_s_sleep(8);
  }
  // (the stamp goes first: once the last counter is out, the consumer may finish and the caller
  // may read the trace)
  if (p.trace) p.trace[c] = wall_clock64();
  if (p.ctr_index[c] >= 0 && (p.pos[c] == 0 || !((p.withhold_mask >> p.pos[c]) & 1u)))
    __hip_atomic_store(ctr + p.ctr_index[c] * kWordStride, epoch, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}

// Start of a launch that runs copies: zero the other set of counts for the next call and stamp
// the start.  Called by every thread.
__device__ inline void copy_queue_begin(const CopyPlan& p) {
  if (blockIdx.x != 0) return;
  if (threadIdx.x < 2 * kArrSlots)
    __hip_atomic_store(p.clear_next + threadIdx.x * kWordStride, 0u, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  if (p.trace && threadIdx.x == 0) p.trace[kTraceStart] = wall_clock64();
}

// Take pieces of queue q (0 = the early peers' chunks, 2 = the late ones, 1 = the own chunk's
// copies) and copy them until the queue
// is empty, until max_pieces are copied or, with stop >= 0, until ctr[stop] == epoch (checked
// before each take).  Called by every thread of the workgroup; s_word is a workgroup-shared word.
//
// Each iteration has exactly one thread-0 step, between barriers: complete the piece copied in
// the previous iteration, then take the next one.  (With a thread-0 step at the end of the body
// and another at the start, the compiler may thread their common condition across the back edge
// and lower the loop so that thread 0's lane is held back while the wave's other lanes start the
// next iteration with the stale piece number, a loop that never ends.)  The taken number is read
// into a scalar register, so the loop's exit is uniform.
template <int NT, int U = 8, bool PIPE = true>
__device__ inline void run_copy_queue(const CopyPlan& p, int* ctr, int epoch, int q, int stop,
                                      unsigned* s_word, unsigned max_pieces = ~0u) {
  const unsigned early = (unsigned)(p.n_peer - p.late);
  const unsigned first = q == 0 ? 0u : q == 1 ? (unsigned)p.n_peer : early;
  const unsigned total =
      (q == 0 ? early : q == 1 ? (unsigned)(p.n - p.n_peer) : (unsigned)p.late) * p.pieces;
  if (total == 0) return;
  unsigned prev = ~0u;   // copy of the piece finished in the previous iteration, if any
  unsigned taken = 0;    // pieces copied (uniform)
  while (true) {
    if (threadIdx.x == 0) {
      if (prev != ~0u) pieces_done(p, ctr, epoch, prev, 1);
      unsigned g = ~0u;
      if (taken < max_pieces &&
          (stop < 0 || __hip_atomic_load(ctr + stop * kWordStride, __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT) != epoch))
        g = __hip_atomic_fetch_add(p.grab + q * kWordStride, 1u, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
      *s_word = g;
    }
    __syncthreads();
    const unsigned g = __builtin_amdgcn_readfirstlane(*s_word);
    __syncthreads();
    if (g >= total) return;
    const unsigned c = first + g / p.pieces;
    copy_piece<NT, U, PIPE>(p, c, g % p.pieces);
    // every wave waits for its own stores; after the barrier thread 0 completes the piece
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    prev = c;
    ++taken;
  }
}

}  // namespace ringag
