// Device-side building blocks of the "TN" GEMM tile used by both operations:
//     out[i][j] = sum_k X[i][k] * Y[j][k]       X [rows, K], Y [cols, K], both K-contiguous
// on gfx950 matrix cores.  A workgroup of WI x WJ waves computes a BI x BJ output tile; wave
// (wi, wj) owns the (BI/WI) x (BJ/WJ) sub-tile at (wi * BI/WI, wj * BJ/WJ), made of 32 x 32 MFMA
// blocks with fp32 accumulators.
//
// Data path per K step (128 bytes of K per row: 64 bf16 or 128 fp8 elements):
//   HBM/L2 --buffer_load_dwordx4 ... lds (16 B per lane, range-checked by the descriptor)--> LDS
//   LDS --ds_read_b128--> VGPR fragments --v_mfma--> accumulators
// LDS holds two stages: while the waves multiply stage s, the loads of stage s^1 are in flight.
// The loads are issued with inline assembly so that the compiler, which cannot tell that they
// write the other stage, does not wait for them before every read of the current one; the code
// waits for them explicitly (vmcnt(0)) at the end of each step, before the barrier that hands the
// stage to the readers.  Rows of 128 bytes are stored with their eight 16-byte segments permuted by
// XOR with ((row >> 1) & 7): gfx950's LDS serves 256 bytes (64 banks) per cycle, i.e. 16 lanes of
// a ds_read_b128, which read 16 consecutive rows at the same logical segment; even and odd rows
// fall in different bank halves and the key gives the 8 rows of each parity 8 distinct segments.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#pragma clang diagnostic ignored "-Winline-asm"

namespace ringag {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr int kRowBytes = 128;                 // bytes of K per row per stage
constexpr uint32_t kOOB = 0x80000000u;         // voffset that is always past num_records

template <int BI_, int BJ_, int WI_, int WJ_>
struct TileShape {
  static constexpr int BI = BI_, BJ = BJ_, WI = WI_, WJ = WJ_;
  static constexpr int NW = WI * WJ;             // waves
  static constexpr int NT = NW * 64;             // threads
  static constexpr int TM = BI / WI, TN = BJ / WJ;   // wave sub-tile
  static constexpr int FI = TM / 32, FJ = TN / 32;   // MFMA blocks per wave
  static constexpr int STAGE = (BI + BJ) * kRowBytes;
  static constexpr int XQ = BI / (8 * NW);       // 8-row load groups of X per wave
  static constexpr int YQ = BJ / (8 * NW);
  // bf16 output staging: rows padded by 16 bytes so the two row halves a wave writes do not
  // share banks
  static constexpr int OUT_LD = BJ * 2 + 16;
  static constexpr int LDS_MAIN = 2 * STAGE;
  static constexpr int LDS_OUT = BI * OUT_LD;
  static constexpr int LDS = LDS_MAIN > LDS_OUT ? LDS_MAIN : LDS_OUT;
  static_assert(BI % (8 * NW) == 0 && BJ % (8 * NW) == 0, "load groups must divide evenly");
  static_assert(TM % 32 == 0 && TN % 32 == 0, "wave tiles are made of 32x32 blocks");
};

using Tile128x128 = TileShape<128, 128, 2, 2>;
using Tile256x128 = TileShape<256, 128, 2, 2>;
using Tile256x256 = TileShape<256, 256, 2, 2>;     // 4 waves of 128x128
using Tile256x256w8 = TileShape<256, 256, 2, 4>;   // 8 waves of 128x64

// Raw buffer descriptor (gfx9 family: base, stride 0, num_records = size in bytes, word 3 =
// 0x00020000).  Loads at offsets >= num_records return zero instead of faulting, which is how
// partial tiles (ragged rows) are read.
__device__ inline i32x4 make_rsrc(const void* p, uint32_t bytes) {
  const uint64_t a = (uint64_t)(uintptr_t)p;
  i32x4 r;
  r[0] = (int)(uint32_t)a;
  r[1] = (int)(uint32_t)(a >> 32);   // stride 0
  r[2] = (int)bytes;
  r[3] = 0x00020000;
  return r;
}

// One 16-byte-per-lane load into LDS: lane l writes LDS bytes [lds + 16 l, lds + 16 l + 16).
__device__ inline void dma16(i32x4 rsrc, uint32_t lds_addr, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(lds_addr), "v"(voff), "s"(rsrc)
               : "memory", "m0");
}

__device__ inline void wait_vmem_all() {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

__device__ inline uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)p;
}

// Swizzle key of a tile row (see the header comment).
__device__ inline int swz(int row) { return (row >> 1) & 7; }

// Per-lane byte offsets (relative to the operand's first row) of the segments this lane loads in
// each of its Q row groups.  Lane l of an 8-row group writes tile row 8 g + l/8 at physical segment
// l%8, so it fetches logical segment (l%8) ^ swz(row).  Rows at or past rows_valid get kOOB
// (zeros).  row0 is a multiple of 16, so tile-local and global rows share their swizzle key.
template <int Q, int NW>
__device__ inline void tile_offsets(uint32_t* voff, int row0, int rows_valid, uint32_t ld_bytes,
                                    int wave, int lane) {
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    const int lr = (q * NW + wave) * 8 + (lane >> 3);
    const int logical = (lane & 7) ^ swz(lr);
    const int r = row0 + lr;
    voff[q] = (r < rows_valid) ? (uint32_t)r * ld_bytes + (uint32_t)logical * 16u : kOOB;
  }
}

template <int Q, int NW>
__device__ inline void issue_loads(i32x4 rsrc, const uint32_t* voff, uint32_t kbytes,
                                   uint32_t lds_tile, int wave) {
#pragma unroll
  for (int q = 0; q < Q; ++q)
    dma16(rsrc, lds_tile + (uint32_t)((q * NW + wave) * 8 * kRowBytes), voff[q] + kbytes);
}

// Load one MFMA operand fragment (32 rows x 16 bytes of K per lane half) from a swizzled tile.
// tile_rows is at a multiple of 32 rows, so the lane's row key is swz(lane & 31).
__device__ inline bf16x8 frag_bf16(const char* tile_rows, int seg_logical, int lane) {
  const int r = lane & 31;
  return *(const bf16x8*)(tile_rows + r * kRowBytes + ((seg_logical ^ swz(r)) << 4));
}

__device__ inline i32x8 frag_fp8(const char* tile_rows, int seg_logical, int lane) {
  const int r = lane & 31;
  const char* row = tile_rows + r * kRowBytes;
  const i32x4 lo = *(const i32x4*)(row + ((seg_logical ^ swz(r)) << 4));
  const i32x4 hi = *(const i32x4*)(row + (((seg_logical + 1) ^ swz(r)) << 4));
  return (i32x8){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// Multiply one stage held in LDS.  bf16: 4 MFMA k-steps of 16 (v_mfma_f32_32x32x16_bf16); fp8
// E4M3: 2 k-steps of 64 (v_mfma_scale_f32_32x32x64_f8f6f4 with unit scales).  Lane l of a 32x32
// operand fragment holds row (l & 31) and the (l >> 5)-th half of the k-step; X (MFMA A operand,
// output rows) and Y (B operand, output columns) use the same k assignment.
template <class S, bool FP8>
__device__ inline void stage_mma(const char* xs, const char* ys, int lane,
                                 f32x16 (&acc)[S::FI][S::FJ]) {
  const int h = lane >> 5;
  if constexpr (!FP8) {
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      bf16x8 a[S::FI], b[S::FJ];
#pragma unroll
      for (int f = 0; f < S::FI; ++f) a[f] = frag_bf16(xs + f * 32 * kRowBytes, kk * 2 + h, lane);
#pragma unroll
      for (int f = 0; f < S::FJ; ++f) b[f] = frag_bf16(ys + f * 32 * kRowBytes, kk * 2 + h, lane);
#pragma unroll
      for (int i = 0; i < S::FI; ++i)
#pragma unroll
        for (int j = 0; j < S::FJ; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
  } else {
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      i32x8 a[S::FI], b[S::FJ];
#pragma unroll
      for (int f = 0; f < S::FI; ++f) a[f] = frag_fp8(xs + f * 32 * kRowBytes, kk * 4 + h * 2, lane);
#pragma unroll
      for (int f = 0; f < S::FJ; ++f) b[f] = frag_fp8(ys + f * 32 * kRowBytes, kk * 4 + h * 2, lane);
#pragma unroll
      for (int i = 0; i < S::FI; ++i)
#pragma unroll
        for (int j = 0; j < S::FJ; ++j)
          // format 0 = FP8 E4M3 for both operands; E8M0 scale 127 = 2^0 on both
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[i], b[j], acc[i][j], 0, 0,
                                                                      0, 127, 0, 127);
    }
  }
}

// Full K loop of one tile.  rx/ry: descriptors of X and Y; xo/yo from tile_offsets; ksteps = K
// bytes / 128.  Returns with acc = the wave's fp32 sub-tile and all waves past a final barrier
// (LDS free for the epilogue).  The caller must have passed a barrier since the last LDS reads.
template <class S, bool FP8>
__device__ inline void tile_kloop(i32x4 rx, const uint32_t* xo, i32x4 ry, const uint32_t* yo,
                                  int ksteps, char* lds, int wave, int lane,
                                  f32x16 (&acc)[S::FI][S::FJ]) {
  const int wi = wave / S::WJ, wj = wave % S::WJ;
  const uint32_t base = lds_addr(lds);
#pragma unroll
  for (int i = 0; i < S::FI; ++i)
#pragma unroll
    for (int j = 0; j < S::FJ; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  issue_loads<S::XQ, S::NW>(rx, xo, 0, base, wave);
  issue_loads<S::YQ, S::NW>(ry, yo, 0, base + S::BI * kRowBytes, wave);
  wait_vmem_all();
  __syncthreads();
  for (int kt = 0; kt < ksteps; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < ksteps) {
      const uint32_t kb = (uint32_t)(kt + 1) * kRowBytes;
      const uint32_t nxt = base + (uint32_t)((cur ^ 1) * S::STAGE);
      issue_loads<S::XQ, S::NW>(rx, xo, kb, nxt, wave);
      issue_loads<S::YQ, S::NW>(ry, yo, kb, nxt + S::BI * kRowBytes, wave);
    }
    const char* st = lds + cur * S::STAGE;
    stage_mma<S, FP8>(st + wi * S::TM * kRowBytes, st + (S::BI + wj * S::TN) * kRowBytes, lane,
                      acc);
    wait_vmem_all();
    __syncthreads();
  }
}

// Output coordinates of accumulator element e of block (i, j) for this lane, relative to the
// wave's sub-tile origin: row = 32 i + 8 (e / 4) + 4 (lane / 32) + e % 4, col = 32 j + lane % 32.
__device__ inline int acc_row(int i, int e, int lane) {
  return i * 32 + (e >> 2) * 8 + (lane >> 5) * 4 + (e & 3);
}
__device__ inline int acc_col(int j, int lane) { return j * 32 + (lane & 31); }

// Epilogue for bf16 output: the accumulators (times `scale`) are rounded to bf16 into an LDS
// tile, then written out row by row with 16-byte stores (whole 64-byte+ row segments per group of
// lanes).  out points at row 0 of the tile's rows; ld = row stride in elements; rows/cols valid =
// how much of the tile lies inside the output.  Ends with a barrier (LDS free again).
template <class S>
__device__ inline void store_tile_bf16(const f32x16 (&acc)[S::FI][S::FJ], float scale, char* lds,
                                       __bf16* out, int ld, int rows_valid, int cols_valid,
                                       int wave, int lane) {
  const int wi = wave / S::WJ, wj = wave % S::WJ;
#pragma unroll
  for (int i = 0; i < S::FI; ++i)
#pragma unroll
    for (int j = 0; j < S::FJ; ++j) {
      const int col = wj * S::TN + acc_col(j, lane);
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int row = wi * S::TM + acc_row(i, e, lane);
        *(__bf16*)(lds + row * S::OUT_LD + col * 2) = (__bf16)(acc[i][j][e] * scale);
      }
    }
  __syncthreads();
  constexpr int SEGS = S::BJ / 8;   // 16-byte segments per tile row
  const bool vec = (ld % 8) == 0 && (((uintptr_t)out) & 15u) == 0;
  for (int idx = threadIdx.x; idx < S::BI * SEGS; idx += S::NT) {
    const int r = idx / SEGS, sg = idx % SEGS;
    const int c = sg * 8;
    if (r >= rows_valid || c >= cols_valid) continue;
    const char* src = lds + r * S::OUT_LD + c * 2;
    __bf16* dst = out + (size_t)r * ld + c;
    if (vec && c + 8 <= cols_valid) {
      *(i32x4*)dst = *(const i32x4*)src;
    } else {
      for (int e = 0; e < 8 && c + e < cols_valid; ++e) dst[e] = ((const __bf16*)src)[e];
    }
  }
  __syncthreads();
}

}  // namespace ringag
