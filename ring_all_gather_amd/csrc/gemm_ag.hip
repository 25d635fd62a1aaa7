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

template <class S, bool FP8>
__global__ void __launch_bounds__(S::NT) ag_gemm_kernel(AgArgs a) {
  __shared__ __attribute__((aligned(1024))) char lds[S::LDS];
  __shared__ int s_ok;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t ldb = (uint32_t)a.K * (FP8 ? 1u : 2u);
  const int ksteps = (int)(ldb / kRowBytes);
  const int U = a.tiles_i * a.tiles_j;
  const int total = U * a.tp;
  float scale = 1.0f;
  if constexpr (FP8) scale = a.scale_A[0] * a.scale_B[0];
  const i32x4 ry = make_rsrc(a.A, (uint32_t)a.M * ldb);

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
    const i32x4 rx = make_rsrc(a.chunk[j], (uint32_t)a.nc * ldb);
    uint32_t xo[S::XQ], yo[S::YQ];
    tile_offsets<S::XQ, S::NW>(xo, rb * S::BI, a.nc, ldb, wave, lane);
    tile_offsets<S::YQ, S::NW>(yo, cb * S::BJ, a.M, ldb, wave, lane);
    f32x16 acc[S::FI][S::FJ];
    tile_kloop<S, FP8>(rx, xo, ry, yo, ksteps, lds, wave, lane, acc);
    __bf16* out = (__bf16*)a.out[j] + (size_t)rb * S::BI * a.M + (size_t)cb * S::BJ;
    store_tile_bf16<S>(acc, scale, lds, out, a.M, a.nc - rb * S::BI, a.M - cb * S::BJ, wave, lane);
  }
}

template <class S, bool FP8>
static hipError_t launch_t(const AgArgs& a, int grid, hipStream_t s) {
  hipLaunchKernelGGL((ag_gemm_kernel<S, FP8>), dim3(grid), dim3(S::NT), 0, s, a);
  return hipGetLastError();
}

template <class S, bool FP8>
static hipError_t info_t(KernelInfo* info) {
  hipFuncAttributes at;
  hipError_t e = hipFuncGetAttributes(&at, (const void*)ag_gemm_kernel<S, FP8>);
  if (e != hipSuccess) return e;
  int nb = 0;
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, ag_gemm_kernel<S, FP8>, S::NT, 0);
  if (e != hipSuccess) return e;
  info->threads = S::NT;
  info->lds_bytes = (int)at.sharedSizeBytes;
  info->vgprs_per_wave = at.numRegs;
  info->max_blocks_per_cu = nb;
  return hipSuccess;
}

template <class S>
static hipError_t launch_dt(const AgArgs& a, bool fp8, int grid, hipStream_t s) {
  return fp8 ? launch_t<S, true>(a, grid, s) : launch_t<S, false>(a, grid, s);
}

template <class S>
static hipError_t info_dt(bool fp8, KernelInfo* info) {
  return fp8 ? info_t<S, true>(info) : info_t<S, false>(info);
}

hipError_t launch_ag_gemm(const AgArgs& a, int tile, bool fp8, int grid, hipStream_t s) {
  switch (tile) {
    case kTile256x256: return launch_dt<Tile256x256>(a, fp8, grid, s);
    case kTile256x256w8: return launch_dt<Tile256x256w8>(a, fp8, grid, s);
    case kTile256x128: return launch_dt<Tile256x128>(a, fp8, grid, s);
    default: return launch_dt<Tile128x128>(a, fp8, grid, s);
  }
}

hipError_t ag_kernel_info(int tile, bool fp8, KernelInfo* info) {
  switch (tile) {
    case kTile256x256: return info_dt<Tile256x256>(fp8, info);
    case kTile256x256w8: return info_dt<Tile256x256w8>(fp8, info);
    case kTile256x128: return info_dt<Tile256x128>(fp8, info);
    default: return info_dt<Tile128x128>(fp8, info);
  }
}

}  // namespace ringag
