// Device-side building blocks of the "TN" GEMM tile used by both operations:
//     out[i][j] = sum_k X[i][k] * Y[j][k]       X [rows, K], Y [cols, K], both K-contiguous
// on gfx950 matrix cores.  One workgroup = 4 waves (2 x 2) computes a BI x BJ output tile; each
// wave owns a (BI/2) x (BJ/2) sub-tile made of 32 x 32 MFMA blocks with fp32 accumulators.
//
// Data path per K step (BK bytes of K per row = 128 bytes: 64 bf16 or 128 fp8 elements):
//   HBM/L2 --buffer_load ... lds (16 B per lane, bounds-checked by the buffer descriptor)--> LDS
//   LDS --ds_read_b128--> VGPR fragments --v_mfma--> accumulators
// LDS holds two stages (double buffering): while the waves multiply stage s, the loads for stage
// s^1 are in flight.  Rows of 128 bytes are stored with their eight 16-byte segments permuted by
// XOR with (row & 7), so that the 32 rows one MFMA operand read touches spread over all banks.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ringag {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kRowBytes = 128;                 // bytes of K per row per stage
constexpr uint32_t kOOB = 0x80000000u;         // voffset that is always past num_records

// Buffer descriptor over [p, p + bytes): loads at offsets >= bytes return zero instead of
// faulting, which is how partial tiles (ragged rows) are read.  Word 3 = 0x00020000 is the
// gfx9-family raw-buffer format used for plain 32-bit-dword loads.
__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}

__device__ inline lds_void_t* to_lds(void* p) {
  return (lds_void_t*)(p);
}

// Issue the loads of one operand tile (ROWS rows x 128 bytes) into LDS.  Lane l of a wave
// instruction writes LDS bytes [l*16, l*16+16) past the instruction's base, i.e. row l/8 of an
// 8-row group at physical segment l%8; it therefore fetches logical segment (l%8) ^ (l/8).
// voff[q] is the lane's byte offset of that segment in row-group q (kOOB for rows past the end).
template <int ROWS>
__device__ inline void issue_tile_loads(__amdgpu_buffer_rsrc_t rsrc, const uint32_t* voff,
                                        uint32_t kbytes, char* lds_tile, int wave) {
#pragma unroll
  for (int q = 0; q < ROWS / 32; ++q) {
    const int g = q * kWaves + wave;                     // 8-row group index
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, to_lds(lds_tile + g * 8 * kRowBytes), 16,
                                             voff[q] + kbytes, 0, 0, 0);
  }
}

// Per-lane byte offsets (relative to the operand's first row) of the segments this lane loads.
template <int ROWS>
__device__ inline void tile_offsets(uint32_t* voff, int row0, int rows_valid, uint32_t ld_bytes,
                                    int wave, int lane) {
  const int lrow = lane >> 3;
  const int logical = (lane & 7) ^ lrow;
#pragma unroll
  for (int q = 0; q < ROWS / 32; ++q) {
    const int r = row0 + (q * kWaves + wave) * 8 + lrow;
    voff[q] = (r < rows_valid) ? (uint32_t)r * ld_bytes + (uint32_t)logical * 16u : kOOB;
  }
}

__device__ inline void wait_vmem_all() {
  // s_waitcnt vmcnt(0), leaving expcnt/lgkmcnt unconstrained (gfx9 encoding)
  __builtin_amdgcn_s_waitcnt(0x0F70);
}

// Accumulate one stage (128 bytes of K) of the tile from LDS.
// FP8 = false: bf16, 4 MFMA k-steps of 16 (v_mfma_f32_32x32x16_bf16).
// FP8 = true : E4M3, 2 MFMA k-steps of 64 (v_mfma_scale_f32_32x32x64_f8f6f4, unit scales).
// Lane l of a 32x32 operand fragment holds row (l & 31) and the (l >> 5)-th half of the k-step;
// A (rows of X) and B (rows of Y) use the same k assignment, so their products pair correctly.
template <int FI, int FJ, bool FP8>
__device__ inline void stage_mma(const char* lds_x, const char* lds_y, int lane,
                                 f32x16 (&acc)[FI][FJ]) {
  const int r = lane & 31;
  const int h = lane >> 5;
  const int sw = lane & 7;     // rows of a fragment start at multiples of 8, so row & 7 == lane & 7
  if constexpr (!FP8) {
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int seg = ((kk * 2 + h) ^ sw) * 16;
      bf16x8 a[FI], b[FJ];
#pragma unroll
      for (int f = 0; f < FI; ++f)
        a[f] = *(const bf16x8*)(lds_x + (f * 32 + r) * kRowBytes + seg);
#pragma unroll
      for (int f = 0; f < FJ; ++f)
        b[f] = *(const bf16x8*)(lds_y + (f * 32 + r) * kRowBytes + seg);
#pragma unroll
      for (int i = 0; i < FI; ++i)
#pragma unroll
        for (int j = 0; j < FJ; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
  } else {
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int s0 = ((kk * 4 + h * 2) ^ sw) * 16;
      const int s1 = ((kk * 4 + h * 2 + 1) ^ sw) * 16;
      i32x8 a[FI], b[FJ];
#pragma unroll
      for (int f = 0; f < FI; ++f) {
        const char* p = lds_x + (f * 32 + r) * kRowBytes;
        i32x4 lo = *(const i32x4*)(p + s0);
        i32x4 hi = *(const i32x4*)(p + s1);
        a[f] = (i32x8){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      }
#pragma unroll
      for (int f = 0; f < FJ; ++f) {
        const char* p = lds_y + (f * 32 + r) * kRowBytes;
        i32x4 lo = *(const i32x4*)(p + s0);
        i32x4 hi = *(const i32x4*)(p + s1);
        b[f] = (i32x8){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      }
#pragma unroll
      for (int i = 0; i < FI; ++i)
#pragma unroll
        for (int j = 0; j < FJ; ++j)
          // format 0 = FP8 E4M3 for both operands; E8M0 scale 127 = 2^0 on both
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[i], b[j], acc[i][j], 0, 0,
                                                                      0, 127, 0, 127);
    }
  }
}

// Full K loop of one BI x BJ tile.  rx/ry: descriptors of X and Y; x_voff/y_voff from
// tile_offsets; ksteps = K bytes / 128.  On return acc holds the wave's fp32 sub-tile.
// LDS: 2 stages of (BI + BJ) * 128 bytes.  The caller must have passed a barrier since the last
// reads of this LDS (the loop ends with one).
template <int BI, int BJ, bool FP8>
__device__ inline void tile_kloop(__amdgpu_buffer_rsrc_t rx, const uint32_t* x_voff,
                                  __amdgpu_buffer_rsrc_t ry, const uint32_t* y_voff, int ksteps,
                                  char* lds, int wave, int lane,
                                  f32x16 (&acc)[BI / 64][BJ / 64]) {
  constexpr int FI = BI / 64, FJ = BJ / 64;
  constexpr int STAGE = (BI + BJ) * kRowBytes;
  const int wi = wave >> 1, wj = wave & 1;
#pragma unroll
  for (int i = 0; i < FI; ++i)
#pragma unroll
    for (int j = 0; j < FJ; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  issue_tile_loads<BI>(rx, x_voff, 0, lds, wave);
  issue_tile_loads<BJ>(ry, y_voff, 0, lds + BI * kRowBytes, wave);
  wait_vmem_all();
  __syncthreads();
  for (int kt = 0; kt < ksteps; ++kt) {
    char* cur = lds + (kt & 1) * STAGE;
    char* nxt = lds + ((kt & 1) ^ 1) * STAGE;
    if (kt + 1 < ksteps) {
      const uint32_t kb = (uint32_t)(kt + 1) * kRowBytes;
      issue_tile_loads<BI>(rx, x_voff, kb, nxt, wave);
      issue_tile_loads<BJ>(ry, y_voff, kb, nxt + BI * kRowBytes, wave);
    }
    stage_mma<FI, FJ, FP8>(cur + wi * (BI / 2) * kRowBytes,
                           cur + BI * kRowBytes + wj * (BJ / 2) * kRowBytes, lane, acc);
    wait_vmem_all();
    __syncthreads();
  }
}

// Output coordinates of accumulator element e of fragment (i, j) for this lane, relative to the
// wave's sub-tile origin: row = 32 i + 8 (e / 4) + 4 (lane / 32) + e % 4, col = 32 j + lane % 32.
__device__ inline int acc_row(int i, int e, int lane) {
  return i * 32 + (e >> 2) * 8 + (lane >> 5) * 4 + (e & 3);
}
__device__ inline int acc_col(int j, int lane) { return j * 32 + (lane & 31); }

}  // namespace ringag
