// GEMM + reduce-scatter kernel (row-parallel linear, one rank's share).
//
// TransformerEngine PR #2443, sequence diagram: the RS path splits the GEMM and reduce-scatters
// its output; review comments: the contraction dimension of that GEMM is the local shard of a
// global k.  nvFuser PR #5742, walkthrough: each chunk of the output is summed over ranks.
//
// The rank computes its whole partial P = X W^T, chunk by chunk in ring order (the rank's own
// chunk last, as in a ring reduce-scatter where the own chunk's sum completes last).  Tiles of
// another rank's chunk store their fp32 accumulators to `send` (the outgoing contribution).
// Tiles of the own chunk add the peers' fp32 partials to the accumulators while they are still in
// registers and store the bf16 result: the reduction costs no extra pass over D.
#pragma once

#include "gemm_core.hpp"
#include "kernels.hpp"

namespace ringag {

template <class S>
__device__ __forceinline__ void gemm_rs_body(const RsArgs& a) {
  __shared__ __attribute__((aligned(1024))) char lds[S::LDS];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wi = wave / S::WJ, wj = wave % S::WJ;
  const uint32_t ldb = (uint32_t)a.Kl * 2u;
  const int ksteps = (int)(ldb / S::BKB);
  const int U = a.tiles_i * a.tiles_j;
  const int total = U * a.tp;
  const i32x4 ry = make_rsrc(a.W, (uint32_t)a.Mo * ldb);

  for (int t = blockIdx.x; t < total; t += gridDim.x) {
    const int j = t / U;
    const int u = t - j * U;
    const int c = a.chunk_of[j];
    const bool own = (c == a.self_rank);
    if (!own && a.send == nullptr) continue;
    int rb, cb;
    map_tile_xcd(u, U, a.tiles_i, a.tiles_j, a.xcd_rows, &rb, &cb);
    const char* xbase = (const char*)a.X + (size_t)c * a.nc * ldb;
    const i32x4 rx = make_rsrc(xbase, (uint32_t)a.nc * ldb);
    uint32_t xo[S::XQ], yo[S::YQ];
    tile_offsets<S, S::XQ>(xo, rb * S::BI, a.nc, ldb, wave, lane);
    tile_offsets<S, S::YQ>(yo, cb * S::BJ, a.Mo, ldb, wave, lane);
    f32x16 acc[S::FI][S::FJ];
    tile_kloop<S, false>(rx, xo, ry, yo, ksteps, lds, wave, lane, acc);

    const int row0 = rb * S::BI + wi * S::TM;
    const int col0 = cb * S::BJ + wj * S::TN;
    if (!own) {
      float* out = a.send + (size_t)c * a.nc * a.Mo;
#pragma unroll
      for (int i = 0; i < S::FI; ++i)
#pragma unroll
        for (int jj = 0; jj < S::FJ; ++jj) {
          const int col = col0 + acc_col(jj, lane);
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int row = row0 + acc_row(i, e, lane);
            if (row < a.nc && col < a.Mo) out[(size_t)row * a.Mo + col] = acc[i][jj][e];
          }
        }
    } else {
      // Own chunk: add every peer's partial to the accumulators one block at a time (16 extra
      // registers live), then round to bf16 and store.
      __bf16* out = (__bf16*)a.D;
      const size_t prow0 = (size_t)a.self_rank * a.nc;
#pragma unroll
      for (int i = 0; i < S::FI; ++i)
#pragma unroll
        for (int jj = 0; jj < S::FJ; ++jj) {
          const int col = col0 + acc_col(jj, lane);
          float v[16];
#pragma unroll
          for (int e = 0; e < 16; ++e) v[e] = acc[i][jj][e];
          for (int p = 0; p < a.tp; ++p) {
            if (p == a.self_rank) continue;
            const float* part = a.partial[p] + prow0 * (size_t)a.ldp;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
              const int row = row0 + acc_row(i, e, lane);
              if (row < a.nc && col < a.Mo) v[e] += part[(size_t)row * a.ldp + col];
            }
          }
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int row = row0 + acc_row(i, e, lane);
            if (row < a.nc && col < a.Mo) out[(size_t)row * a.Mo + col] = (__bf16)v[e];
          }
        }
    }
  }
}

}  // namespace ringag
