// Counter-gated AG+GEMM kernel (the consumer side of the ring all-gather).
//
// TransformerEngine issue #1583, C++ listing: one GEMM launch, split into tp pieces along the
// gathered dimension, consumes chunk after chunk; before touching a chunk it waits for that
// chunk's counter, which the receive side bumps after each ring step.  Here the launch is a
// persistent grid; tile t of the ring-ordered tile sequence (all tiles of the own chunk, then all
// tiles of the first chunk to arrive, ...) runs on workgroup t mod grid.  A tile's first wave polls
// its chunk's counter (agent-scope acquire, bounded by a wall-clock limit), the workgroup meets at
// a barrier, and the K loop starts.  Each chunk's output rows go straight to that chunk's rank
// offset of D (or to its staging slot), so D is rank-ordered for every self rank.
//
// With in-kernel copies (AgArgs::copies) the launch also carries the call's arrival: a workgroup
// whose next tile belongs to a chunk that is not there yet takes pieces of the peers' chunks from
// the copy queue (ring order) until that chunk is released, and once out of tiles it helps with
// whatever is left, the own chunk's copy into G last.  The waiting workgroups are the ones with
// nothing to compute yet (in a one-round launch the own chunk's workgroups, which have time to
// spare, also copy one piece each first), so the copies use compute units that would otherwise
// idle, and no side stream or stream fork/join is involved.
//
// With K-slab gating (AgArgs::slab, bf16 8-wave 2-stage tiles) the peers' chunks are not queued
// whole: every workgroup copies its own slots of slab pieces (before its first tile, inside its K
// loops, after its last tile), and a tile waits only for the slab its next loads read; see
// slab_copy.hpp.
#pragma once

#include "copy_queue.hpp"
#include "gemm_core.hpp"
#include "kernels.hpp"
#include "slab_copy.hpp"

namespace ringag {

// (XCC << 16) | (shader engine << 8) | CU of the calling wave (hardware id registers).
__device__ inline unsigned hw_location() {
  const unsigned xcc = __builtin_amdgcn_s_getreg((3 << 11) | (0 << 6) | 20);   // XCC_ID[3:0]
  const unsigned se = __builtin_amdgcn_s_getreg((1 << 11) | (13 << 6) | 4);    // HW_ID[14:13]
  const unsigned cu = __builtin_amdgcn_s_getreg((3 << 11) | (8 << 6) | 4);     // HW_ID[11:8]
  return (xcc << 16) | (se << 8) | cu;
}

template <class T>
struct TileTag {
  using type = T;
};

// The half tile of an 8-wave 256-column tile: the same rows and waves, half the columns, each
// wave 64x64.  A round of the persistent grid that is at most half full (the last one of a
// problem whose tile count is not a multiple of the grid) runs its tiles as two halves on two
// workgroups, so that every compute unit works through it instead of half of them for a whole
// tile time.  ag_fc1_f8 (896 tiles, 3.5 rounds): chunked call 401 -> 391 us, GEMM-only 365 ->
// 359 us (one box); less than the half round's share, since half-idle rounds ran at a higher
// clock.
template <class S>
struct HalfTile {
  static constexpr bool on = S::NW == 8 && S::BJ == 256 && S::BKB == 128 && S::NS == 2;
  using type = TileShape<S::BI, 128, 4, 2, S::BKB, S::NS>;
};

// SLAB: the K-slab-gated form (its own entry points, so that the registers and LDS of the slab
// copies are not charged to the chunk-gated kernels).
template <class S, bool FP8, bool OUT8, bool SLAB = false>
__device__ __forceinline__ void ag_gemm_body(const AgArgs& a) {
  static_assert(!SLAB || (!FP8 && S::NT == kSlabThreads && S::NS == 2 && S::BKB == 128),
                "K-slab gating is built for bf16 8-wave tiles with 2 stages of 128 bytes");
  __shared__ __attribute__((aligned(1024))) char lds[S::LDS];
  __shared__ int s_ok;
  __shared__ unsigned s_piece;
  __shared__ int s_gate;
  __shared__ __attribute__((aligned(1024))) char s_slab[SLAB ? kSlabMaxQ * 8192 : 16];
  __shared__ float s_red[OUT8 ? S::NW : 1];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t ldb = (uint32_t)a.K * (FP8 ? 1u : 2u);
  const int ksteps = (int)(ldb / S::BKB);
  const int U = a.tiles_i * a.tiles_j;
  const int total = U * a.tp;
  float scale = 1.0f;
  if constexpr (FP8) scale = a.scale_A[0] * a.scale_B[0];
  const i32x4 ry = make_rsrc(a.A, (uint32_t)a.M * ldb);
  if (a.copies) copy_queue_begin(a.cp);
  const bool copier = a.copies && ((blockIdx.x >> 3) % a.copy_stride) == 0;
  // the software-pipelined copy holds two register sets; the 4-wave 256x256 tile (128x128 per
  // wave, 256 accumulator registers) spills without them already, so it copies with the plain loop
  constexpr bool kPipe = !(S::NW == 4 && S::FI * S::FJ >= 16);
  constexpr bool slab = SLAB;
  int slot = 0;   // slab gating: this workgroup's next slot of pieces
  if (slab) {
    slab_copy_slots(a, 0, a.slab.pre, ldb);
    slot = a.slab.pre;
  }

  const int grid = (int)gridDim.x;
  for (int r0 = 0; a.compute && r0 < total; r0 += grid) {
    const int n = min(grid, total - r0);
    // a round at most half full runs as 2n half tiles (HalfTile), dealt like whole ones
    const bool split = HalfTile<S>::on && !SLAB && 2 * n <= grid;
    int t, half = 0;
    if (split) {
      const int v = round_tile(0, 2 * n, grid);
      if (v < 0) continue;
      t = r0 + (v >> 1);
      half = v & 1;
    } else {
      t = round_tile(r0, n, grid);
      if (t < 0) continue;
    }
    const int j = t / U;
    const int u = t - j * U;
    const int rb = u % a.tiles_i, cb = u / a.tiles_i;
    // (one stamp record per tile: a split tile's first half writes it)
    unsigned long long* tr =
        a.trace && half == 0 ? a.trace + kTraceTileWords * (size_t)t : nullptr;
    if (tr && threadIdx.x == 0) tr[0] = wall_clock64();
    // In a one-round launch the own chunk's tiles start at once and end well before the peers'
    // tiles, which start only after the copies; so each of the own chunk's workgroups first
    // copies one piece of the peers' chunks.  The copies then run on every XCD, not only on those
    // holding the peers' tiles, and each XCD's path to memory carries less of them (ag_4k chunked
    // call 112.5-113.0 -> 111.5-112.0 us, one box).  With more rounds the delay reaches the own
    // workgroups' later tiles (ag_fc1_f8 394.0-394.5 -> 395.5-396.6 us), so they do not.
    if (copier && !slab && total <= grid && a.ctr_index[j] < 0) {
      run_copy_queue<S::NT, 8, kPipe>(a.cp, a.ctr, a.epoch, 0, -1, &s_piece, 1u);
      __syncthreads();   // keeps the queue's thread-0 step and this tile's apart
    }
    if (slab && a.ctr_index[j] >= 0) {
      slab_gate_tile(a, j - 1, ldb, &s_gate);
    } else if (a.ctr_index[j] >= 0) {
      if (copier) {
        run_copy_queue<S::NT, 8, kPipe>(a.cp, a.ctr, a.epoch, 0, a.ctr_index[j], &s_piece);
        if (!a.cp.late_external)
          run_copy_queue<S::NT, 8, kPipe>(a.cp, a.ctr, a.epoch, 2, a.ctr_index[j], &s_piece);
      }
      if (threadIdx.x == 0)
        s_ok = wait_ready(a.ctr + a.ctr_index[j] * kWordStride, a.epoch, a.err, a.spin_limit);
      __syncthreads();
      const int ok = __builtin_amdgcn_readfirstlane(s_ok);   // uniform: see run_copy_queue
      __syncthreads();
      if (!ok) continue;
    }
    unsigned long long cyc0 = 0;
    if (tr && threadIdx.x == 0) {
      tr[1] = wall_clock64();
      cyc0 = __builtin_amdgcn_s_memtime();
    }
    const i32x4 rx = make_rsrc(a.chunk[j], (uint32_t)a.nc * ldb);
    // the tile (or half tile) of shape T whose first output column is col0
    auto run_tile = [&](auto tag, int col0) {
      using T = typename decltype(tag)::type;
      uint32_t xo[T::XQ], yo[T::YQ];
      tile_offsets<T, T::XQ>(xo, rb * T::BI, a.nc, ldb, wave, lane);
      tile_offsets<T, T::YQ>(yo, col0, a.M, ldb, wave, lane);
      f32x16 acc[T::FI][T::FJ];
      if constexpr (SLAB) {
        SlabHook hook{a, a.ctr_index[j] >= 0 ? j - 1 : -1, ksteps, ldb, &s_gate, s_slab, slot};
        tile_kloop_bf16<T>(rx, xo, ry, yo, ksteps, lds, wave, lane, acc, hook);
      } else {
        tile_kloop<T, FP8>(rx, xo, ry, yo, ksteps, lds, wave, lane, acc);
      }
      if constexpr (OUT8) {
        uint8_t* out = (uint8_t*)a.out[j] + (size_t)rb * T::BI * a.M + (size_t)col0;
        const float m = store_tile_fp8<T, acc_block<T, FP8>()>(
            acc, scale, a.scale_D[0], lds, out, a.M, a.nc - rb * T::BI, a.M - col0, wave, lane);
        if (a.amax_D) {
          const float bm = block_max<T>(m, s_red, wave, lane);
          // amax >= 0, so its bits order like unsigned integers (a NaN sorts above everything)
          if (threadIdx.x == 0)
            __hip_atomic_fetch_max((unsigned*)a.amax_D, __float_as_uint(bm), __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
        }
      } else {
        __bf16* out = (__bf16*)a.out[j] + (size_t)rb * T::BI * a.M + (size_t)col0;
        store_tile_bf16<T, acc_block<T, FP8>()>(acc, scale, lds, out, a.M, a.nc - rb * T::BI,
                                               a.M - col0, wave, lane);
      }
    };
    if constexpr (HalfTile<S>::on && !SLAB) {
      using Th = typename HalfTile<S>::type;
      if (split) {
        // (a right half wholly past the last column has nothing to do)
        if (cb * S::BJ + half * Th::BJ < a.M) run_tile(TileTag<Th>{}, cb * S::BJ + half * Th::BJ);
      } else {
        run_tile(TileTag<S>{}, cb * S::BJ);
      }
    } else {
      run_tile(TileTag<S>{}, cb * S::BJ);
    }
    if (tr && threadIdx.x == 0) {
      tr[2] = wall_clock64();
      tr[3] = ((unsigned long long)blockIdx.x << 32) | hw_location();
      tr[4] = __builtin_amdgcn_s_memtime() - cyc0;
    }
    // keeps this thread-0 step and the next tile's apart (see run_copy_queue)
    __syncthreads();
  }
  if (slab) slab_copy_slots(a, slot, max(slot, slab_slots_end(a)), ldb);
  if (copier) {
    if (!slab) {
      run_copy_queue<S::NT, 8, kPipe>(a.cp, a.ctr, a.epoch, 0, -1, &s_piece);
      if (!a.cp.late_external)
        run_copy_queue<S::NT, 8, kPipe>(a.cp, a.ctr, a.epoch, 2, -1, &s_piece);
    }
    run_copy_queue<S::NT, 8, kPipe>(a.cp, a.ctr, a.epoch, 1, -1, &s_piece);
  }
  // With the copies on another stream, which the caller's stream does not wait for, the kernel
  // ends only once the last copy (the own chunk into G) is complete, so that everything enqueued
  // after it sees a complete G.  The peers' chunks are complete already, since some tile waited
  // for each of them.
  if (a.join_index >= 0 && threadIdx.x == 0)
    (void)wait_ready(a.ctr + a.join_index * kWordStride, a.epoch, a.err, a.spin_limit);
}

}  // namespace ringag
