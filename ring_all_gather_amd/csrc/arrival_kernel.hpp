// Arrival (producer) kernel: stands in for the receive side of the ring on one GPU.
//
// TransformerEngine issue #1583, C++ listing: on the receive stream, each ring step copies one
// chunk into the gathered buffer and then marks it ready with a per-chunk counter ("producer");
// the listing's multi-atomic variant does all steps in one launch.  This kernel is that one-launch
// form: its workgroups copy the chunks one after another in ring order, and once a chunk is
// complete its counter is released with the call's epoch, so the GEMM tiles of that chunk start
// while the next chunk is still being copied.
//
// Work is handed out dynamically: a chunk is cut into pieces of kArrPiece bytes and each workgroup
// takes the next piece with an atomic until none is left, so workgroups that share a compute unit
// with busy GEMM waves simply copy less (a static split would make every chunk wait for its
// slowest slice).  Each workgroup then adds the number of pieces it copied to the chunk's done
// count with one agent-scope release (writing its XCD's L2 back), and the workgroup whose addition
// completes the count releases the chunk's counter.  The grab and done counts come in two sets
// used by alternate launches; a launch clears the other set for the next one (launches of one
// context are ordered on its side stream, so the next launch sees the cleared set).  The kernel
// needs no LDS beyond two words and few registers, so its waves fit beside the GEMM's.
#pragma once

#include <hip/hip_runtime.h>

#include "kernels.hpp"

namespace ringag {

typedef int v4i __attribute__((ext_vector_type(4)));

constexpr int kArrThreads = kArrivalThreads;
constexpr int kArrUnroll = 8;
constexpr unsigned long long kArrPiece = 64 * 1024;   // bytes per grab

__device__ __forceinline__ void arrival_body(const ArrivalArgs& a) {
  __shared__ unsigned long long s_piece;
  // The copy shares SIMDs with GEMM waves: issue its (few) instructions first so the chunks the
  // GEMM waits for are not starved by the waves that will consume them.
  if (a.raise_priority) __builtin_amdgcn_s_setprio(3);
  if (a.trace && blockIdx.x == 0 && threadIdx.x == 0) a.trace[kTraceStart] = wall_clock64();
  if (blockIdx.x == 0 && threadIdx.x < 2 * kArrSlots)
    __hip_atomic_store(a.clear_next + threadIdx.x * kWordStride, 0u, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);

  const unsigned long long pieces = (a.bytes + kArrPiece - 1) / kArrPiece;
  for (int j = 0; j < a.n; ++j) {
    const char* src = (const char*)a.src[j];
    char* dst = (char*)a.dst[j];
    unsigned mine = 0;
    while (true) {
      if (threadIdx.x == 0)
        s_piece = __hip_atomic_fetch_add(a.grab + j * kWordStride, 1u, __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT);
      __syncthreads();
      const unsigned long long p = s_piece;
      __syncthreads();
      if (p >= pieces) break;
      const unsigned long long beg = p * kArrPiece;
      const unsigned long long len = min(kArrPiece, a.bytes - beg);
      const v4i* s = (const v4i*)(src + beg);
      v4i* d = (v4i*)(dst + beg);
      const unsigned long long nvec = len / 16;
      unsigned long long i = threadIdx.x;
      for (; i + (kArrUnroll - 1) * kArrThreads < nvec; i += kArrUnroll * kArrThreads) {
        v4i v[kArrUnroll];
#pragma unroll
        for (int u = 0; u < kArrUnroll; ++u) v[u] = s[i + u * kArrThreads];
#pragma unroll
        for (int u = 0; u < kArrUnroll; ++u) d[i + u * kArrThreads] = v[u];
      }
      for (; i < nvec; i += kArrThreads) d[i] = s[i];
      ++mine;
    }

    if (a.ctr_index[j] >= 0 && mine > 0) {
      // Each wave waits for its own stores to be acknowledged; after the barrier, one release
      // (agent scope: writes the XCD's L2 back) by thread 0 covers the whole workgroup's pieces.
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      if (threadIdx.x == 0) {
        const unsigned old = __hip_atomic_fetch_add(a.done + j * kWordStride, mine,
                                                    __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
        if (old + mine == (unsigned)pieces) {
          if (a.delay_ticks > 0) {
            const unsigned long long t0 = wall_clock64();
            while ((long long)(wall_clock64() - t0) < a.delay_ticks) __builtin_amdgcn_s_sleep(8);
          }
          // (the stamp goes first: once the last counter is out, the consumer may finish and
          // the caller may read the trace)
          if (a.trace) a.trace[j] = wall_clock64();
          if (a.pos[j] == 0 || !((a.withhold_mask >> a.pos[j]) & 1u))
            __hip_atomic_store(a.ctr + a.ctr_index[j] * kWordStride, a.epoch, __ATOMIC_RELEASE,
                               __HIP_MEMORY_SCOPE_AGENT);
        }
      }
    }
  }
}

}  // namespace ringag
