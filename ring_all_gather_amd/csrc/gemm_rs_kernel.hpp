// GEMM + reduce-scatter kernel (row-parallel linear, one rank's share).
//
// TransformerEngine PR #2443, sequence diagram: the RS path splits the GEMM and reduce-scatters
// its output; review comments: the contraction dimension of that GEMM is the local shard of a
// global k.  nvFuser PR #5742, walkthrough: each chunk of the output is summed over ranks.
//
// The rank computes its whole partial P = X W^T, chunk by chunk in ring order (the rank's own
// chunk last).  One-shot form: tiles of another rank's chunk store their fp32 accumulators to
// `send` (the outgoing contribution); tiles of the own chunk add the peers' fp32 partials of it
// and store the bf16 result.  Ring-accumulate form: the tiles of chunk c add the running sum of c
// that arrives from the previous rank (none for the chunk whose chain starts here) and store the
// result to send, or, for the own chunk, to D.  When that data arrives during the call (gated),
// a tile runs its K loop first and waits for the counters only before its epilogue reads it.
//
// Epilogue: the accumulators are staged through LDS one wave row (TM rows of the tile) at a time,
// then every thread moves whole 16-byte vectors along tile rows: send is written, and partials
// are read, in full contiguous rows rather than in the MFMA layout's 4-byte scatter.  A thread
// holds a batch of vectors and issues one peer's loads for the whole batch before adding them,
// so a batch's loads are in flight together.
#pragma once

#include "copy_queue.hpp"
#include "gemm_core.hpp"
#include "kernels.hpp"

namespace ringag {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

template <class S>
struct RsEpilogue {
  static constexpr int LD = S::BJ * 4 + 32;        // staging row stride: the two rows a wave
                                                    // writes at once fall in different banks
  static constexpr int VPR = S::BJ / 4;            // 16-byte vectors per tile row
  static constexpr int VPT = S::TM * VPR / S::NT;  // vectors per thread per staged wave row
  // 8-wave tiles have half the registers per lane, and the waves of the second wave row still
  // hold their accumulators while the first is reduced: smaller batches there
  static constexpr int MAXB = S::NW >= 8 ? 4 : 8;
  static constexpr int BATCH = VPT < MAXB ? VPT : MAXB;
  static_assert(S::TM * LD <= S::LDS, "a wave row of fp32 accumulators must fit in LDS");
  static_assert((S::TM * VPR) % S::NT == 0 && VPT % BATCH == 0, "vectors must divide evenly");
};

template <class S>
__device__ inline void rs_epilogue(const f32x16 (&acc)[S::FI][S::FJ], char* lds, const RsArgs& a,
                                   int c, bool own, int rb, int cb, int wave, int lane) {
  using E = RsEpilogue<S>;
  const int wi = wave / S::WJ, wj = wave % S::WJ;
  const int col0 = cb * S::BJ;
  for (int slab = 0; slab < S::WI; ++slab) {
    if (wi == slab) {
#pragma unroll
      for (int i = 0; i < S::FI; ++i)
#pragma unroll
        for (int j = 0; j < S::FJ; ++j) {
          const int col = wj * S::TN + acc_col(j, lane);
#pragma unroll
          for (int e = 0; e < 16; ++e)
            *(float*)(lds + acc_row(i, e, lane) * E::LD + col * 4) = acc[i][j][e];
        }
    }
    __syncthreads();
    const int row0 = rb * S::BI + slab * S::TM;   // chunk-local row of the staged row 0
    // what the staged rows get added to: every peer's partial (own chunk, one-shot), one
    // incoming running sum (ring step), or nothing (another chunk, one-shot)
    const int nadd = a.ring ? (a.partial[c] != nullptr ? 1 : 0) : (own ? a.tp - 1 : 0);
    const bool to_d = own;
    if (nadd == 0 && !to_d) {
      float* out = a.send + (size_t)c * a.nc * a.Mo;
#pragma unroll
      for (int k = 0; k < E::VPT; ++k) {
        const int idx = (int)threadIdx.x + k * S::NT;
        const int r = idx / E::VPR, v = idx % E::VPR;
        const int row = row0 + r, col = col0 + v * 4;
        if (row < a.nc && col < a.Mo)
          *(f32x4*)(out + (size_t)row * a.Mo + col) = *(const f32x4*)(lds + r * E::LD + v * 16);
      }
    } else {
      for (int b = 0; b < E::VPT; b += E::BATCH) {
        f32x4 x[E::BATCH];
        int row[E::BATCH], col[E::BATCH];
        bool ok[E::BATCH];
#pragma unroll
        for (int q = 0; q < E::BATCH; ++q) {
          const int idx = (int)threadIdx.x + (b + q) * S::NT;
          const int r = idx / E::VPR, v = idx % E::VPR;
          row[q] = row0 + r;
          col[q] = col0 + v * 4;
          ok[q] = row[q] < a.nc && col[q] < a.Mo;
          x[q] = *(const f32x4*)(lds + r * E::LD + v * 16);
        }
        for (int i = 0; i < nadd; ++i) {
          // one-shot: the i-th peer in increasing rank, skipping this rank; ring: chunk c's sum
          const int p = a.ring ? c : (i < a.self_rank ? i : i + 1);
          const float* part = a.partial[p];
          f32x4 y[E::BATCH];
#pragma unroll
          for (int q = 0; q < E::BATCH; ++q) {
            const float* src = part + (size_t)row[q] * a.ldp + col[q];
            if (!ok[q]) y[q] = f32x4{0.f, 0.f, 0.f, 0.f};
            else if (a.partial_vec) y[q] = *(const f32x4*)src;
            else y[q] = f32x4{src[0], src[1], src[2], src[3]};
          }
#pragma unroll
          for (int q = 0; q < E::BATCH; ++q) x[q] += y[q];
        }
        if (to_d) {
          __bf16* out = (__bf16*)a.D;
#pragma unroll
          for (int q = 0; q < E::BATCH; ++q)
            if (ok[q])
              *(bf16x4*)(out + (size_t)row[q] * a.Mo + col[q]) =
                  bf16x4{(__bf16)x[q][0], (__bf16)x[q][1], (__bf16)x[q][2], (__bf16)x[q][3]};
        } else {
          float* out = a.send + (size_t)c * a.nc * a.Mo;
#pragma unroll
          for (int q = 0; q < E::BATCH; ++q)
            if (ok[q]) *(f32x4*)(out + (size_t)row[q] * a.Mo + col[q]) = x[q];
        }
      }
    }
    __syncthreads();
  }
}

template <class S>
__device__ __forceinline__ void gemm_rs_body(const RsArgs& a) {
  __shared__ __attribute__((aligned(1024))) char lds[S::LDS];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t ldb = (uint32_t)a.Kl * 2u;
  const int ksteps = (int)(ldb / S::BKB);
  const int U = a.tiles_i * a.tiles_j;
  const int total = U * a.tp;
  const i32x4 ry = make_rsrc(a.W, (uint32_t)a.Mo * ldb);
  const int grid = (int)gridDim.x;
  __shared__ int s_ok;

  for (int r0 = 0; r0 < total; r0 += grid) {
    const int t = round_tile(r0, min(grid, total - r0), grid);
    if (t < 0) continue;
    const int j = t / U;
    const int u = t - j * U;
    const int c = a.chunk_of[j];
    const bool own = (c == a.self_rank);
    if (!own && a.send == nullptr) continue;
    const int rb = u % a.tiles_i, cb = u / a.tiles_i;
    const char* xbase = (const char*)a.X + (size_t)c * a.nc * ldb;
    const i32x4 rx = make_rsrc(xbase, (uint32_t)a.nc * ldb);
    uint32_t xo[S::XQ], yo[S::YQ];
    tile_offsets<S, S::XQ>(xo, rb * S::BI, a.nc, ldb, wave, lane);
    tile_offsets<S, S::YQ>(yo, cb * S::BJ, a.Mo, ldb, wave, lane);
    f32x16 acc[S::FI][S::FJ];
    tile_kloop<S, false>(rx, xo, ry, yo, ksteps, lds, wave, lane, acc);
    // gated: wait for what the epilogue reads (the K loop did not need it)
    const bool waits = a.gated && (a.ring ? a.partial[c] != nullptr : own);
    if (waits) {
      if (threadIdx.x == 0) {
        bool ok = true;
        if (a.ring) {
          ok = wait_ready(a.ctr + c * kWordStride, a.epoch, a.err, a.spin_limit);
        } else {
          for (int p = 0; p < a.tp && ok; ++p)
            if (p != a.self_rank)
              ok = wait_ready(a.ctr + p * kWordStride, a.epoch, a.err, a.spin_limit);
        }
        s_ok = ok;
      }
      __syncthreads();
      const int ok = __builtin_amdgcn_readfirstlane(s_ok);   // uniform: see run_copy_queue
      __syncthreads();
      if (!ok) continue;
    }
    rs_epilogue<S>(acc, lds, a, c, own, rb, cb, wave, lane);
  }
}

}  // namespace ringag
