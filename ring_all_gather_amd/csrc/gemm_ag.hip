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
#include "gemm_core.hpp"
#include "kernels.hpp"

namespace ringag {

// Chunk-local tile u -> (row block, column block).  Workgroups are dealt round-robin to the 8 XCDs
// (each with its own L2), so tile u runs on XCD u % 8 when the grid and the chunk's tile count are
// multiples of 8.  The permutation gives each XCD a contiguous run of column blocks with every row
// block of the chunk: the XCD's L2 then serves one slab of the weight and the chunk's rows.
__device__ inline void map_tile(int u, int U, int R, int* rb, int* cb) {
  int v = u;
  if ((U & 7) == 0) v = (u & 7) * (U >> 3) + (u >> 3);
  *rb = v % R;
  *cb = v / R;
}

// Wait until *ctr == epoch.  Returns false when the limit passed or another tile of this call
// already gave up (then *err == epoch).
__device__ inline bool wait_ready(int* ctr, int epoch, int* err, long long limit) {
  if (__hip_atomic_load(ctr, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT) == epoch) return true;
  const unsigned long long t0 = wall_clock64();
  while (true) {
    __builtin_amdgcn_s_sleep(2);
    if (__hip_atomic_load(ctr, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT) == epoch) return true;
    if (__hip_atomic_load(err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == epoch) return false;
    if ((long long)(wall_clock64() - t0) > limit) {
      __hip_atomic_store(err, epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return false;
    }
  }
}

template <int BI, int BJ, bool FP8>
__global__ void __launch_bounds__(kThreads) ag_gemm_kernel(AgArgs a) {
  __shared__ __attribute__((aligned(1024))) char lds[2 * (BI + BJ) * kRowBytes];
  __shared__ int s_ok;
  constexpr int FI = BI / 64, FJ = BJ / 64;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wi = wave >> 1, wj = wave & 1;
  const uint32_t ldb = (uint32_t)a.K * (FP8 ? 1u : 2u);
  const int ksteps = (int)(ldb / kRowBytes);
  const int U = a.tiles_i * a.tiles_j;
  const int total = U * a.tp;
  float scale = 1.0f;
  if constexpr (FP8) scale = a.scale_A[0] * a.scale_B[0];
  const __amdgpu_buffer_rsrc_t ry = make_rsrc(a.A, (uint32_t)a.M * ldb);

  for (int t = blockIdx.x; t < total; t += gridDim.x) {
    const int j = t / U;
    const int u = t - j * U;
    int rb, cb;
    map_tile(u, U, a.tiles_i, &rb, &cb);
    if (a.ctr_index[j] >= 0) {
      if (threadIdx.x == 0) s_ok = wait_ready(a.ctr + a.ctr_index[j], a.epoch, a.err, a.spin_limit);
      __syncthreads();
      const int ok = s_ok;
      __syncthreads();
      if (!ok) continue;
    }
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(a.chunk[j], (uint32_t)a.nc * ldb);
    uint32_t xo[BI / 32], yo[BJ / 32];
    tile_offsets<BI>(xo, rb * BI, a.nc, ldb, wave, lane);
    tile_offsets<BJ>(yo, cb * BJ, a.M, ldb, wave, lane);
    f32x16 acc[FI][FJ];
    tile_kloop<BI, BJ, FP8>(rx, xo, ry, yo, ksteps, lds, wave, lane, acc);

    __bf16* out = (__bf16*)a.out[j];
    const int row0 = rb * BI + wi * (BI / 2);
    const int col0 = cb * BJ + wj * (BJ / 2);
#pragma unroll
    for (int i = 0; i < FI; ++i)
#pragma unroll
      for (int jj = 0; jj < FJ; ++jj) {
        const int col = col0 + acc_col(jj, lane);
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int row = row0 + acc_row(i, e, lane);
          if (row < a.nc && col < a.M)
            out[(size_t)row * a.M + col] = (__bf16)(acc[i][jj][e] * scale);
        }
      }
  }
}

template <int BI, int BJ, bool FP8>
static hipError_t launch_t(const AgArgs& a, int grid, hipStream_t s) {
  hipLaunchKernelGGL((ag_gemm_kernel<BI, BJ, FP8>), dim3(grid), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

template <int BI, int BJ, bool FP8>
static hipError_t info_t(KernelInfo* info) {
  hipFuncAttributes at;
  hipError_t e = hipFuncGetAttributes(&at, (const void*)ag_gemm_kernel<BI, BJ, FP8>);
  if (e != hipSuccess) return e;
  int nb = 0;
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, ag_gemm_kernel<BI, BJ, FP8>, kThreads, 0);
  if (e != hipSuccess) return e;
  info->threads = kThreads;
  info->lds_bytes = (int)at.sharedSizeBytes;
  info->vgprs_per_wave = at.numRegs;
  info->max_blocks_per_cu = nb;
  return hipSuccess;
}

hipError_t launch_ag_gemm(const AgArgs& a, int tile, bool fp8, int grid, hipStream_t s) {
  switch (tile) {
    case kTile256x256: return fp8 ? launch_t<256, 256, true>(a, grid, s)
                                  : launch_t<256, 256, false>(a, grid, s);
    case kTile256x128: return fp8 ? launch_t<256, 128, true>(a, grid, s)
                                  : launch_t<256, 128, false>(a, grid, s);
    default: return fp8 ? launch_t<128, 128, true>(a, grid, s)
                        : launch_t<128, 128, false>(a, grid, s);
  }
}

hipError_t ag_kernel_info(int tile, bool fp8, KernelInfo* info) {
  switch (tile) {
    case kTile256x256: return fp8 ? info_t<256, 256, true>(info) : info_t<256, 256, false>(info);
    case kTile256x128: return fp8 ? info_t<256, 128, true>(info) : info_t<256, 128, false>(info);
    default: return fp8 ? info_t<128, 128, true>(info) : info_t<128, 128, false>(info);
  }
}

}  // namespace ringag
