// Arrival (producer) kernel: stands in for the receive side of the ring on one GPU.
//
// TransformerEngine issue #1583, C++ listing: on the receive stream, each ring step copies one
// chunk into the gathered buffer and then marks it ready with a per-chunk counter ("producer");
// the listing's multi-atomic variant does all steps in one launch.  This kernel is that one-launch
// form: its workgroups copy the chunks one after another in ring order, each workgroup taking a
// contiguous slice of every chunk; the last workgroup to finish a chunk (a self-resetting ticket)
// releases the chunk's counter with the call's epoch, so tiles of that chunk can start while the
// next chunk is still being copied.  It needs no LDS and few registers, so its waves fit beside
// the GEMM's on every compute unit.
#pragma once

#include <hip/hip_runtime.h>

#include "kernels.hpp"

namespace ringag {

typedef int v4i __attribute__((ext_vector_type(4)));

constexpr int kArrThreads = kArrivalThreads;
constexpr int kArrUnroll = 8;

__device__ __forceinline__ void arrival_body(const ArrivalArgs& a) {
  const unsigned long long nvec = a.bytes / 16;
  const unsigned long long per = (nvec + gridDim.x - 1) / gridDim.x;
  const unsigned long long beg = min(nvec, (unsigned long long)blockIdx.x * per);
  const unsigned long long end = min(nvec, beg + per);
  // The copy shares SIMDs with GEMM waves: issue its (few) instructions first so the chunks the
  // GEMM waits for are not starved by the waves that will consume them.
  if (a.raise_priority) __builtin_amdgcn_s_setprio(3);
  if (a.trace && blockIdx.x == 0 && threadIdx.x == 0) a.trace[kTraceStart] = wall_clock64();
  for (int j = 0; j < a.n; ++j) {
    const v4i* src = (const v4i*)a.src[j];
    v4i* dst = (v4i*)a.dst[j];
    unsigned long long i = beg + threadIdx.x;
    for (; i + (kArrUnroll - 1) * kArrThreads < end; i += kArrUnroll * kArrThreads) {
      v4i v[kArrUnroll];
#pragma unroll
      for (int u = 0; u < kArrUnroll; ++u) v[u] = src[i + u * kArrThreads];
#pragma unroll
      for (int u = 0; u < kArrUnroll; ++u) dst[i + u * kArrThreads] = v[u];
    }
    for (; i < end; i += kArrThreads) dst[i] = src[i];

    if (a.ctr_index[j] >= 0) {
      // Each wave waits for its own stores to be acknowledged; after the barrier, one release
      // (agent scope: writes the XCD's L2 back) by thread 0 covers the whole workgroup's slice.
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      if (threadIdx.x == 0) {
        const int old = __hip_atomic_fetch_add(a.ticket + j, 1, __ATOMIC_ACQ_REL,
                                               __HIP_MEMORY_SCOPE_AGENT);
        if (old == (int)gridDim.x - 1) {
          __hip_atomic_store(a.ticket + j, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          if (a.delay_ticks > 0) {
            const unsigned long long t0 = wall_clock64();
            while ((long long)(wall_clock64() - t0) < a.delay_ticks) __builtin_amdgcn_s_sleep(8);
          }
          if (!((a.withhold_mask >> a.pos[j]) & 1u))
            __hip_atomic_store(a.ctr + a.ctr_index[j], a.epoch, __ATOMIC_RELEASE,
                               __HIP_MEMORY_SCOPE_AGENT);
          if (a.trace) a.trace[j] = wall_clock64();
        }
      }
    }
  }
}

}  // namespace ringag
