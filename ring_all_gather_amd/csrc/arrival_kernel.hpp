// Arrival (producer) kernel: stands in for the receive side of the ring on one GPU.
//
// TransformerEngine issue #1583, C++ listing: on the receive stream, each ring step copies one
// chunk into the gathered buffer and then marks it ready with a per-chunk counter ("producer");
// the listing's multi-atomic variant does all steps in one launch.  This kernel is that one-launch
// form on the library's side stream: its workgroups run the call's piece queue (copy_queue.hpp) in
// ring order, so the GEMM tiles of a chunk start while later chunks are still being copied.
// Pieces are handed out dynamically, so workgroups that share a compute unit with busy GEMM waves
// simply copy less.  The kernel needs no LDS beyond one word and few registers, so its waves fit
// beside the GEMM's.
#pragma once

#include "copy_queue.hpp"

namespace ringag {

// 16-byte vectors in flight per copying thread: 6 keeps the kernel at 38 VGPRs (40 as allocated),
// which fit beside two GEMM waves of up to 232 VGPRs on a SIMD (of its 512).
constexpr int kArrivalInFlight = 6;

__device__ __forceinline__ void arrival_body(const ArrivalArgs& a) {
  __shared__ unsigned s_piece;
  // The copy shares SIMDs with GEMM waves: issue its (few) instructions first so the chunks the
  // GEMM waits for are not starved by the waves that will consume them.
  if (a.raise_priority) __builtin_amdgcn_s_setprio(3);
  copy_queue_begin(a.cp);
  if (!a.late_only)
    run_copy_queue<kArrivalThreads, kArrivalInFlight, false>(a.cp, a.ctr, a.epoch, 0, -1,
                                                             &s_piece);
  run_copy_queue<kArrivalThreads, kArrivalInFlight, false>(a.cp, a.ctr, a.epoch, 2, -1,
                                                           &s_piece);
  run_copy_queue<kArrivalThreads, kArrivalInFlight, false>(a.cp, a.ctr, a.epoch, 1, -1,
                                                           &s_piece);
}

}  // namespace ringag
