// Internal interface between the host runtime (runtime.cpp) and the kernel translation units.
// Nothing here is part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ringag {

constexpr int kMaxTp = 16;

// Arguments of the counter-gated AG+GEMM kernel.  Chunk positions j = 0..tp-1 are the ring order
// at this rank (position 0 = own chunk).
struct AgArgs {
  const void* chunk[kMaxTp];     // by position: where the kernel reads that chunk's rows
  void* out[kMaxTp];             // by position: where that chunk's [nc, M] bf16 output rows go
  int ctr_index[kMaxTp];         // by position: counter to wait for, -1 = ready from the start
  const void* A;                 // weight [M, K]
  int M, K, nc, tp;
  int* ctr;                      // per-chunk ready counters
  int epoch;                     // value meaning "ready" for this call
  int* err;                      // error word: set to 1 when a wait times out
  long long spin_limit;          // wall-clock ticks a tile waits before giving up
  const float* scale_A;          // fp8: dequantisation factors (device scalars)
  const float* scale_B;
  int tiles_i, tiles_j;          // tile grid of one chunk
};

// Arguments of the GEMM+RS kernel.  Row-chunk positions j = 0..tp-1 in visiting order; the last
// one is this rank's own chunk, whose tiles are reduced with the peers' partials.
struct RsArgs {
  const void* X;                 // [T, Kl] bf16
  const void* W;                 // [Mo, Kl] bf16
  int chunk_of[kMaxTp];          // by position: row chunk index c
  const float* partial[kMaxTp];  // by rank: peers' fp32 partials (row stride ldp); self unused
  long long ldp;
  float* send;                   // [tp, nc, Mo] fp32 or null
  void* D;                       // [nc, Mo] bf16
  int T, Kl, Mo, nc, tp, self_rank;
  int tiles_i, tiles_j;
};

// Arguments of the arrival (producer) kernel: copies j = 0..n-1 in order, each followed (when
// ctr_index[j] >= 0) by a release of ctr[ctr_index[j]] = epoch once every workgroup finished it.
struct ArrivalArgs {
  const void* src[kMaxTp + 1];
  void* dst[kMaxTp + 1];
  int ctr_index[kMaxTp + 1];
  int pos[kMaxTp + 1];           // ring position of copy j (for the withhold mask)
  int n;
  unsigned long long bytes;      // bytes per copy, multiple of 16
  int* ctr;
  int* ticket;                   // one per copy, self-resetting
  int epoch;
  long long delay_ticks;         // test hook: hold each release back this long
  unsigned withhold_mask;        // test hook: bit pos set = never release that chunk
};

enum TileCfg { kTile128x128 = 1, kTile256x128 = 2, kTile256x256 = 3, kTile256x256w8 = 4 };

struct KernelInfo {
  int threads;
  int lds_bytes;
  int vgprs_per_wave;   // arch + acc registers, as reported by the runtime
  int max_blocks_per_cu;
};

// Launchers: enqueue on `stream`, return hipError_t of the launch.
hipError_t launch_ag_gemm(const AgArgs& a, int tile, bool fp8, int grid, hipStream_t stream);
hipError_t launch_gemm_rs(const RsArgs& a, int tile, int grid, hipStream_t stream);
hipError_t launch_arrival(const ArrivalArgs& a, int grid, hipStream_t stream);

// Occupancy / resource facts for a kernel variant (cached by the caller).
hipError_t ag_kernel_info(int tile, bool fp8, KernelInfo* info);
hipError_t rs_kernel_info(int tile, KernelInfo* info);
hipError_t arrival_kernel_info(KernelInfo* info);

// Tile sizes of a configuration.
inline void tile_dims(int tile, int* bi, int* bj) {
  switch (tile) {
    case kTile256x256:
    case kTile256x256w8: *bi = 256; *bj = 256; break;
    case kTile256x128: *bi = 256; *bj = 128; break;
    default: *bi = 128; *bj = 128; break;
  }
}

}  // namespace ringag
