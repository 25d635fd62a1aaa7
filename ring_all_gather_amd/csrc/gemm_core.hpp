// Device-side building blocks of the "TN" GEMM tile used by both operations:
//     out[i][j] = sum_k X[i][k] * Y[j][k]       X [rows, K], Y [cols, K], both K-contiguous
// on gfx950 matrix cores.  A workgroup of WI x WJ waves computes a BI x BJ output tile; wave
// (wi, wj) owns the (BI/WI) x (BJ/WJ) sub-tile at (wi * BI/WI, wj * BJ/WJ), held as 32 x 32
// blocks of fp32 accumulators, which the K loop fills with 32x32 MFMAs or, four 16x16 blocks
// each, with 16x16 MFMAs (acc_row / acc_col give the layout).
//
// Data path per K step (BKB bytes of K per row: 64 or 128 bytes, i.e. 32/64 bf16 or 64/128 fp8):
//   HBM/L2 --buffer_load_dwordx4 ... lds (16 B per lane, range-checked by the descriptor)--> LDS
//   LDS --ds_read_b128--> VGPR fragments --v_mfma--> accumulators
// LDS holds NS stages in a ring: while the waves multiply stage s, the loads of later stages are
// in flight.  The loads are issued with inline assembly: the compiler cannot tell which stage they
// write, and would otherwise wait for all of them before every LDS read.  Their completion is
// awaited explicitly with s_waitcnt vmcnt(N), N = the loads issued after the stage about to be
// read, followed by the one barrier per stage, which also tells the loads issued after it that the
// stage they overwrite has been read.  Where that wait and barrier sit inside the stage, and how
// the loads and fragment reads are spread over the MFMAs, is the K loop's business: see
// tile_kloop_bf16, tile_kloop_bf16_32 and tile_kloop_2s_fp8 (the pipelined loops) and tile_kloop
// (the plain one, for the 4-stage fp8 tile).
//
// LDS layout: rows of BKB bytes, split into 16-byte segments whose order is permuted by an XOR
// key of the row (swz).  gfx950's LDS serves 256 bytes (64 banks) per cycle, i.e. 16 lanes of a
// ds_read_b128; an MFMA operand read has those 16 lanes on 16 consecutive rows at the same logical
// segment, and the key spreads them over all 64 banks.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#pragma clang diagnostic ignored "-Winline-asm"

namespace ringag {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr uint32_t kOOB = 0x80000000u;         // voffset that is always past num_records

// Accumulator layouts (the MB parameter of acc_row / acc_col and the epilogues): kAcc32 after
// 32x32 MFMAs; kAcc16 after 16x16 MFMAs, four 16x16 blocks per 32x32 block of the array;
// kAcc16S = kAcc16 after acc_swap_rows16.
constexpr int kAcc32 = 32, kAcc16 = 16, kAcc16S = 17;

template <int BI_, int BJ_, int WI_, int WJ_, int BKB_, int NS_>
struct TileShape {
  static constexpr int BI = BI_, BJ = BJ_, WI = WI_, WJ = WJ_;
  static constexpr int BKB = BKB_;               // bytes of K per row per stage
  static constexpr int NS = NS_;                 // LDS stages
  static constexpr int NW = WI * WJ;             // waves
  static constexpr int NT = NW * 64;             // threads
  static constexpr int TM = BI / WI, TN = BJ / WJ;   // wave sub-tile
  static constexpr int FI = TM / 32, FJ = TN / 32;   // MFMA blocks per wave
  static constexpr int SEGS = BKB / 16;          // 16-byte segments per row
  static constexpr int RPI = 1024 / BKB;         // rows written by one 64-lane DMA instruction
  static constexpr int STAGE = (BI + BJ) * BKB;
  static constexpr int XQ = BI / (RPI * NW);     // DMA instructions per wave per stage (X)
  static constexpr int YQ = BJ / (RPI * NW);
  static constexpr int LOADS = XQ + YQ;          // vmcnt increments per wave per stage
  // bf16 output staging row stride, by accumulator layout (store_tile_bf16): rows padded by 16
  // bytes after 16x16 MFMAs, by 32 after 32x32 ones, so that the lanes of one packed LDS write
  // fall in distinct banks
  static constexpr int OUT_LD = BJ * 2 + 16;
  static constexpr int OUT_LD32 = BJ * 2 + 32;
  static constexpr int LDS_MAIN = NS * STAGE;
  static constexpr int LDS_OUT = BI * OUT_LD32;
  static constexpr int LDS = LDS_MAIN > LDS_OUT ? LDS_MAIN : LDS_OUT;
  static_assert(BKB == 64 || BKB == 128, "rows of 64 or 128 bytes");
  static_assert(NS >= 2 && NS <= 4, "2 to 4 stages");
  static_assert(BI % (RPI * NW) == 0 && BJ % (RPI * NW) == 0, "load groups must divide evenly");
  static_assert(TM % 32 == 0 && TN % 32 == 0, "wave tiles are made of 32x32 blocks");
  static_assert((NS - 2) * LOADS <= 63, "vmcnt field holds at most 63");
  static_assert(LDS <= 160 * 1024, "gfx950 has 160 KiB of LDS per workgroup");
};

// The configurations the kernels are built for.
using Tile128x128 = TileShape<128, 128, 2, 2, 128, 2>;
using Tile256x128 = TileShape<256, 128, 2, 2, 128, 2>;
using Tile256x256 = TileShape<256, 256, 2, 2, 128, 2>;      // 4 waves of 128x128, 2 stages
using Tile256x256w8 = TileShape<256, 256, 2, 4, 128, 2>;    // 8 waves of 128x64, 2 stages
using Tile256x256w8s4 = TileShape<256, 256, 2, 4, 64, 4>;   // 8 waves of 128x64, 4 stages
using Tile256x192w8 = TileShape<256, 192, 4, 2, 128, 2>;    // 8 waves of 64x96, 2 stages

// The tile this workgroup runs in the round that covers ring-ordered tiles [r0, r0 + n) of a grid
// of `grid` workgroups, or -1.  Workgroup w runs on XCD w % 8 (workgroups are dealt to the 8 XCDs
// in turn), and XCD x takes the x-th eighth of the round as one contiguous block, so the tiles
// that share an XCD's L2 come from one chunk (or two neighbours in ring order) and are released
// together; tiles from chunks released at different times would share an L2 out of phase and
// fetch the weight's slices separately.  Callers map a chunk-local index u to (u % tiles_i,
// u / tiles_i), so an XCD's block covers all of a chunk's row blocks and a band of the weight's
// rows.  Grids that are not a multiple of 8 use plain round-robin.
__device__ inline int round_tile(int r0, int n, int grid) {
  const int w = (int)blockIdx.x;
  if ((grid & 7) != 0) return w < n ? r0 + w : -1;
  const int x = w & 7, q = w >> 3;
  const int lo = (x * n) >> 3, hi = ((x + 1) * n) >> 3;
  return q < hi - lo ? r0 + lo + q : -1;
}

// Swizzle key of a tile row.  128-byte rows: 2 rows per 256-byte bank line, key (row >> 1) & 7
// gives the 8 rows of each parity in a 16-row group 8 distinct segments.  64-byte rows: 4 rows per
// line, key (row >> 2) & 3 gives the 4 rows of each residue 4 distinct segments.
template <int BKB>
__device__ inline int swz(int row) {
  if constexpr (BKB == 128) return (row >> 1) & 7;
  else return (row >> 2) & 3;
}

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

template <int N>
__device__ inline void wait_vmem() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

__device__ inline uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)p;
}

// Per-lane byte offsets (relative to the operand's first row) of the segment this lane loads in
// each of its Q row groups.  Lane l of a group writes tile row RPI g + l / SEGS at physical segment
// l % SEGS, so it fetches logical segment (l % SEGS) ^ swz(row).  Rows at or past rows_valid get
// kOOB (zeros).  row0 is a multiple of 16, so tile-local and global rows share their key.
template <class S, int Q>
__device__ inline void tile_offsets(uint32_t* voff, int row0, int rows_valid, uint32_t ld_bytes,
                                    int wave, int lane) {
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    const int lr = (q * S::NW + wave) * S::RPI + lane / S::SEGS;
    const int logical = (lane % S::SEGS) ^ swz<S::BKB>(lr);
    const int r = row0 + lr;
    voff[q] = (r < rows_valid) ? (uint32_t)r * ld_bytes + (uint32_t)logical * 16u : kOOB;
  }
}

template <class S, int Q>
__device__ inline void issue_loads(i32x4 rsrc, const uint32_t* voff, uint32_t kbytes,
                                   uint32_t lds_tile, int wave) {
#pragma unroll
  for (int q = 0; q < Q; ++q)
    dma16(rsrc, lds_tile + (uint32_t)((q * S::NW + wave) * S::RPI * S::BKB), voff[q] + kbytes);
}

// One MFMA operand fragment: rows (lane & 31) of a 32-row block starting at tile_rows (a multiple
// of 32 rows into the tile), 16 bytes (bf16) or 32 bytes (fp8) at logical segment `seg`.
template <int BKB>
__device__ inline bf16x8 frag_bf16(const char* tile_rows, int seg, int lane) {
  const int r = lane & 31;
  return *(const bf16x8*)(tile_rows + r * BKB + ((seg ^ swz<BKB>(r)) << 4));
}

template <int BKB>
__device__ inline i32x8 frag_fp8(const char* tile_rows, int seg, int lane) {
  const int r = lane & 31;
  const char* row = tile_rows + r * BKB;
  const i32x4 lo = *(const i32x4*)(row + ((seg ^ swz<BKB>(r)) << 4));
  const i32x4 hi = *(const i32x4*)(row + (((seg + 1) ^ swz<BKB>(r)) << 4));
  return (i32x8){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// Multiply one stage held in LDS.  bf16: k-steps of 16 (v_mfma_f32_32x32x16_bf16); fp8 E4M3:
// k-steps of 64 (v_mfma_scale_f32_32x32x64_f8f6f4 with unit scales).  Lane l of a 32x32 operand
// fragment holds row (l & 31) and the (l >> 5)-th half of the k-step; X (MFMA A operand, output
// rows) and Y (B operand, output columns) use the same k assignment.
//
// bf16 fragments are double-buffered in registers: the reads of k-step kk + 1 are issued before
// the MFMAs of k-step kk (scheduling barriers keep that order), so each read has a k-step of
// MFMAs to land in instead of stalling the wave right before its first use; the LDS latency
// grows while the next stage's DMA writes share the LDS.  (fp8 fragments are twice as large and
// the second set does not fit beside the 8-wave tile's accumulators.)
template <class S, bool FP8>
__device__ inline void stage_mma(const char* xs, const char* ys, int lane,
                                 f32x16 (&acc)[S::FI][S::FJ]) {
  const int h = lane >> 5;
  if constexpr (!FP8) {
    constexpr int NK = S::SEGS / 2;
    bf16x8 a[2][S::FI], b[2][S::FJ];
#pragma unroll
    for (int f = 0; f < S::FI; ++f) a[0][f] = frag_bf16<S::BKB>(xs + f * 32 * S::BKB, h, lane);
#pragma unroll
    for (int f = 0; f < S::FJ; ++f) b[0][f] = frag_bf16<S::BKB>(ys + f * 32 * S::BKB, h, lane);
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) {
      const int c = kk & 1;
      if (kk + 1 < NK) {
#pragma unroll
        for (int f = 0; f < S::FI; ++f)
          a[c ^ 1][f] = frag_bf16<S::BKB>(xs + f * 32 * S::BKB, (kk + 1) * 2 + h, lane);
#pragma unroll
        for (int f = 0; f < S::FJ; ++f)
          b[c ^ 1][f] = frag_bf16<S::BKB>(ys + f * 32 * S::BKB, (kk + 1) * 2 + h, lane);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < S::FI; ++i)
#pragma unroll
        for (int j = 0; j < S::FJ; ++j)
          acc[i][j] =
              __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[c][i], b[c][j], acc[i][j], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  } else {
#pragma unroll
    for (int kk = 0; kk < S::SEGS / 4; ++kk) {
      i32x8 a[S::FI], b[S::FJ];
#pragma unroll
      for (int f = 0; f < S::FI; ++f)
        a[f] = frag_fp8<S::BKB>(xs + f * 32 * S::BKB, kk * 4 + h * 2, lane);
#pragma unroll
      for (int f = 0; f < S::FJ; ++f)
        b[f] = frag_fp8<S::BKB>(ys + f * 32 * S::BKB, kk * 4 + h * 2, lane);
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

// Stage handover inside the K loops: wait until at most N DMA instructions and no LDS reads of
// this wave are outstanding (one instruction; the asm is also a compiler memory barrier), then
// meet the workgroup at the barrier, which the backend keeps ordered with every memory access.
template <int N>
__device__ inline void stage_handover() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"(N) : "memory");
  __builtin_amdgcn_s_barrier();
}

template <class S>
__device__ inline void load_frags_bf16(bf16x8 (&a)[S::FI], bf16x8 (&b)[S::FJ], const char* xs,
                                       const char* ys, int seg, int lane) {
#pragma unroll
  for (int f = 0; f < S::FI; ++f) a[f] = frag_bf16<S::BKB>(xs + f * 32 * S::BKB, seg, lane);
#pragma unroll
  for (int f = 0; f < S::FJ; ++f) b[f] = frag_bf16<S::BKB>(ys + f * 32 * S::BKB, seg, lane);
}

// DMA instructions [q0, q1) of a stage (X rows first, then Y rows) into the stage buffer at byte
// offset buf of the LDS, at K offset kb.
template <class S>
__device__ inline void dma_range(i32x4 rx, const uint32_t* xo, i32x4 ry, const uint32_t* yo,
                                 uint32_t base, int buf, uint32_t kb, int wave, int q0, int q1) {
#pragma unroll
  for (int q = q0; q < q1; ++q) {
    if (q < S::XQ)
      dma16(rx, base + buf + (uint32_t)((q * S::NW + wave) * S::RPI * S::BKB), xo[q] + kb);
    else
      dma16(ry,
            base + buf + S::BI * S::BKB +
                (uint32_t)(((q - S::XQ) * S::NW + wave) * S::RPI * S::BKB),
            yo[q - S::XQ] + kb);
  }
}

// A K loop stage hook that does nothing.
struct NoStageHook {
  __device__ void pre(int) {}
  __device__ void post(int) {}
};

// bf16 K loop with 32x32x16 MFMAs over NS LDS stages (the 64-byte-row tile; the 128-byte-row
// tiles take the 16x16 loop, tile_kloop_bf16 below), with the stage handover inside a stage's
// last MFMA k-step.
// Fragments are double-buffered as in stage_mma.  Once the fragments of the last k-step are in
// registers, the wave waits for its DMA of the next stage and for its reads, meets the others at
// the barrier, reads the next stage's first fragments, and starts the DMA of stage kt + NS into
// the buffer just read.  That DMA is issued in two halves, one DMA instruction after each of a few
// MFMAs: the first half over the last k-step of stage kt, the second over the first k-step of
// stage kt + 1 (all of a stage's DMA in one k-step queues up in the memory pipeline and stalls the
// wave's MFMA issue; spread further, the last pieces have too little time to land).  So no
// fragment read waits right behind a barrier, and the DMA issue hides under MFMAs.  The loop body
// has no branch: past the last stage the DMA reads at kOOB (zeros, into a buffer nobody reads) and
// the prefetch reads an idle buffer; the DMA is drained before the final barrier.  From the
// handover to the start of the next stage a wave issues at raised priority (s_setprio 1), as in
// tile_kloop_bf16 (ag_4k on this tile: GEMM-only 115.8-116.2 -> 113.1-113.5 us, in-GEMM copies
// 128.7-129.7 -> 125.7-126.2 us, one box; all waves at priority 1 gain nothing).
//
// `hook` (see NoStageHook) runs code of the caller's at every stage handover: pre(kt) just before
// the wait and barrier that complete stage kt + 1, post(kt) right after them, before the loads of
// stage kt + 2 are issued.
template <class S, class Hook>
__device__ inline void tile_kloop_bf16_32(i32x4 rx, const uint32_t* xo, i32x4 ry,
                                          const uint32_t* yo, int ksteps, char* lds, int wave,
                                          int lane, f32x16 (&acc)[S::FI][S::FJ], Hook& hook) {
  constexpr int NK = S::SEGS / 2;
  constexpr int NM = S::FI * S::FJ;
  constexpr int H = S::LOADS / 2;   // the first half of a stage's DMA
  static_assert(NK % 2 == 0, "an even number of MFMA k-steps per stage");
  const int wi = wave / S::WJ, wj = wave % S::WJ;
  const int h = lane >> 5;
  const uint32_t base = lds_addr(lds);
#pragma unroll
  for (int i = 0; i < S::FI; ++i)
#pragma unroll
    for (int j = 0; j < S::FJ; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;
  if (ksteps <= 0) {
    __syncthreads();
    return;
  }
  // stages 0 .. NS-2, then (stage 0 complete everywhere) the first half of stage NS-1
#pragma unroll
  for (int st = 0; st < S::NS - 1; ++st) {
    const uint32_t kb = st < ksteps ? (uint32_t)st * S::BKB : kOOB;
    dma_range<S>(rx, xo, ry, yo, base, st * S::STAGE, kb, wave, 0, S::LOADS);
  }
  wait_vmem<(S::NS - 2) * S::LOADS>();
  __syncthreads();
  // the stage whose DMA is under way: its K offset and buffer
  uint32_t pend_kb = S::NS - 1 < ksteps ? (uint32_t)(S::NS - 1) * S::BKB : kOOB;
  int pend_buf = (S::NS - 1) * S::STAGE;
  dma_range<S>(rx, xo, ry, yo, base, pend_buf, pend_kb, wave, 0, H);
  const int xrow = wi * S::TM * S::BKB, yrow = (S::BI + wj * S::TN) * S::BKB;
  bf16x8 a[2][S::FI], b[2][S::FJ];
  load_frags_bf16<S>(a[0], b[0], lds + xrow, lds + yrow, h, lane);
  for (int kt = 0; kt < ksteps; ++kt) {
    const int cur = (S::NS == 2 ? (kt & 1) : kt % S::NS) * S::STAGE;
    const int nxt = S::NS == 2 ? S::STAGE - cur : ((kt + 1) % S::NS) * S::STAGE;
    __builtin_amdgcn_s_setprio(0);
#pragma unroll
    for (int kk = 0; kk < NK - 1; ++kk) {
      const int c = kk & 1;
      load_frags_bf16<S>(a[c ^ 1], b[c ^ 1], lds + cur + xrow, lds + cur + yrow,
                         (kk + 1) * 2 + h, lane);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        const int i = m / S::FJ, j = m % S::FJ;
        acc[i][j] =
            __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[c][i], b[c][j], acc[i][j], 0, 0, 0);
        if (kk == 0) {
          // the second half of the pending stage's DMA, spread over this k-step's MFMAs
          __builtin_amdgcn_sched_barrier(0);
          dma_range<S>(rx, xo, ry, yo, base, pend_buf, pend_kb, wave,
                       H + m * (S::LOADS - H) / NM, H + (m + 1) * (S::LOADS - H) / NM);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // last k-step of the stage (its fragments are in set 1: NK is even).  Outstanding DMA: stages
    // kt+1 .. kt+NS-1, all issued in full; stage kt+1 is complete once at most NS-2 of them are.
    hook.pre(kt);
    stage_handover<(S::NS - 2) * S::LOADS>();
    hook.post(kt);
    __builtin_amdgcn_s_setprio(1);   // until the next stage starts (see above)
    load_frags_bf16<S>(a[0], b[0], lds + nxt + xrow, lds + nxt + yrow, h, lane);
    __builtin_amdgcn_sched_barrier(0);
    pend_kb = kt + S::NS < ksteps ? (uint32_t)(kt + S::NS) * S::BKB : kOOB;
    pend_buf = cur;
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      const int i = m / S::FJ, j = m % S::FJ;
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[1][i], b[1][j], acc[i][j], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
      dma_range<S>(rx, xo, ry, yo, base, pend_buf, pend_kb, wave, m * H / NM, (m + 1) * H / NM);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  __builtin_amdgcn_s_setprio(0);
  wait_vmem<0>();
  __syncthreads();
}

// 16x16x32 MFMA fragment: row (lane & 15) of a 16-row block starting at tile_rows, 16 bytes at
// logical segment `seg` (the lane's quarter of a 32-deep k-step is segment 4 kk + lane / 16).
template <int BKB>
__device__ inline bf16x8 frag16_bf16(const char* tile_rows, int seg, int lane) {
  const int r = lane & 15;
  return *(const bf16x8*)(tile_rows + r * BKB + ((seg ^ swz<BKB>(r)) << 4));
}

// One 16x16x32 MFMA on 16x16 block (gi, gj) of the wave's sub-tile.  The accumulators keep the
// 32x32-block arrays of the other loops: 16x16 block (gi, gj) is elements 4 s .. 4 s + 3 of
// block (gi / 2, gj / 2), s = 2 (gi % 2) + gj % 2 (layout kAcc16 of acc_row / acc_col).
template <int FI, int FJ>
__device__ inline void mma16_bf16(f32x16 (&acc)[FI][FJ], int gi, int gj, const bf16x8& x,
                                  const bf16x8& y) {
  const int i = gi >> 1, j = gj >> 1, s = 2 * (gi & 1) + (gj & 1);
  f32x4 c = {acc[i][j][4 * s], acc[i][j][4 * s + 1], acc[i][j][4 * s + 2], acc[i][j][4 * s + 3]};
  c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x, y, c, 0, 0, 0);
#pragma unroll
  for (int k = 0; k < 4; ++k) acc[i][j][4 * s + k] = c[k];
}

// bf16 K loop for the tiles with two stages of 128-byte rows: 16x16x32 MFMAs, two 32-deep k-steps
// per stage.  The 16x16 shape costs the same MFMA time and LDS traffic as 32x32x16 but runs the
// chip at a higher clock under its power limit (4096^3 GEMM-only, same DMA schedule: 1.81 against
// 1.62 GHz at the same share of busy MFMA cycles).
//
// Per stage kt (fragments of k-step 0 already in set 0):
//   k-step 0: its MFMAs, with the reads of k-step 1 (set 1) placed one after every other MFMA in
//             order of first use;
//   k-step 1: HB MFMAs, then the stage handover (this wave's DMA of stage kt + 1 complete, reads
//             of stage kt done, workgroup barrier), then the rest of its MFMAs with the reads of
//             stage kt + 1's k-step 0 (set 0) and, after each MFMA, a share of the DMA of stage
//             kt + 2 into the buffer of stage kt, which the barrier has freed.
// So the whole DMA of a stage goes out right after a handover and has one full stage to land
// (issued half there and half a k-step later it left the second half short of time: the handover
// then waited on it); no fragment read waits right behind the barrier.  From the handover to the
// start of the next stage a wave issues at raised priority (s_setprio 1): a wave still in that
// part, with its reads and DMA to issue, goes ahead of one on the same SIMD that has already moved
// on to the next stage's MFMAs, so both reach the next barrier sooner (4096^3 GEMM-only 98.6-99.0
// -> 97.4-97.5 us; in the library ag_4k and ag_qkv about 1.2% faster, one box); the loop ends
// at normal priority.  Past the last stage the DMA reads at kOOB (zeros, into a buffer nobody
// reads) and the reads take an idle buffer; the DMA is drained before the final barrier.
// `hook` (see NoStageHook) runs at every handover: pre(kt) right before the wait and barrier that
// complete stage kt + 1, post(kt) right after them, before the loads of stage kt + 2 are issued.
template <class S, class Hook>
__device__ inline void tile_kloop_bf16(i32x4 rx, const uint32_t* xo, i32x4 ry, const uint32_t* yo,
                                       int ksteps, char* lds, int wave, int lane,
                                       f32x16 (&acc)[S::FI][S::FJ], Hook& hook) {
  static_assert(S::BKB == 128 && S::NS == 2, "two stages of 128-byte rows");
  constexpr int GI = 2 * S::FI, GJ = 2 * S::FJ;   // 16x16 blocks of the wave sub-tile
  constexpr int NM = GI * GJ;                     // MFMAs per k-step
  constexpr int NR = GI + GJ;                     // fragment reads per k-step
  constexpr int HB = NM / 4;                      // MFMAs of k-step 1 before the handover
  constexpr int NA = NM - HB;                     // ... and after it
  constexpr int R0 = 2 * NR < NM ? 2 * NR : NM;   // MFMA slots the reads of k-step 1 spread over
  constexpr int R1 = 2 * NR < NA ? 2 * NR : NA;   // ... those of the next stage's k-step 0
  constexpr int L = S::LOADS;
  const int wi = wave / S::WJ, wj = wave % S::WJ;
  const int q4 = lane >> 4;
  const uint32_t base = lds_addr(lds);
#pragma unroll
  for (int i = 0; i < S::FI; ++i)
#pragma unroll
    for (int j = 0; j < S::FJ; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;
  if (ksteps <= 0) {
    __syncthreads();
    return;
  }
  // stage 0, then (stage 0 complete everywhere) stage 1 in full
  dma_range<S>(rx, xo, ry, yo, base, 0, 0, wave, 0, L);
  wait_vmem<0>();
  __syncthreads();
  uint32_t pend_kb = 1 < ksteps ? (uint32_t)S::BKB : kOOB;
  int pend_buf = S::STAGE;
  dma_range<S>(rx, xo, ry, yo, base, pend_buf, pend_kb, wave, 0, L);
  const int xrow = wi * S::TM * S::BKB, yrow = (S::BI + wj * S::TN) * S::BKB;
  bf16x8 a[2][GI], b[2][GJ];
  // read n (in order of first use: x0, y0 .. y(GJ-1), x1 .. x(GI-1)) of the k-step at segment
  // base sg0 of the stage at byte offset st, into fragment set `set`
  auto rd = [&](int set, int st, int n, int sg0) {
    if (n == 0)
      a[set][0] = frag16_bf16<S::BKB>(lds + st + xrow, sg0 + q4, lane);
    else if (n <= GJ)
      b[set][n - 1] = frag16_bf16<S::BKB>(lds + st + yrow + (n - 1) * 16 * S::BKB, sg0 + q4, lane);
    else
      a[set][n - GJ] =
          frag16_bf16<S::BKB>(lds + st + xrow + (n - GJ) * 16 * S::BKB, sg0 + q4, lane);
  };
#pragma unroll
  for (int n = 0; n < NR; ++n) rd(0, 0, n, 0);
  for (int kt = 0; kt < ksteps; ++kt) {
    const int cur = (kt & 1) * S::STAGE;
    const int nxt = S::STAGE - cur;
    __builtin_amdgcn_s_setprio(0);
    // k-step 0 (set 0); reads of k-step 1 (segments 4..7) into set 1
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      mma16_bf16(acc, m / GJ, m % GJ, a[0][m / GJ], b[0][m % GJ]);
      __builtin_amdgcn_sched_barrier(0);
      if (m < R0) {
#pragma unroll
        for (int n = m * NR / R0; n < (m + 1) * NR / R0; ++n) rd(1, cur, n, 4);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // k-step 1 (set 1): HB MFMAs, the handover, the rest with the next stage's first reads and
    // the DMA of stage kt + 2
#pragma unroll
    for (int m = 0; m < HB; ++m) mma16_bf16(acc, m / GJ, m % GJ, a[1][m / GJ], b[1][m % GJ]);
    __builtin_amdgcn_sched_barrier(0);
    hook.pre(kt);
    stage_handover<0>();
    hook.post(kt);
    // raised issue priority until the next stage starts (see above)
    __builtin_amdgcn_s_setprio(1);
    __builtin_amdgcn_sched_barrier(0);
    pend_kb = kt + 2 < ksteps ? (uint32_t)(kt + 2) * S::BKB : kOOB;
    pend_buf = cur;
#pragma unroll
    for (int m = HB; m < NM; ++m) {
      mma16_bf16(acc, m / GJ, m % GJ, a[1][m / GJ], b[1][m % GJ]);
      __builtin_amdgcn_sched_barrier(0);
      const int r = m - HB;
      if (r < R1) {
#pragma unroll
        for (int n = r * NR / R1; n < (r + 1) * NR / R1; ++n) rd(0, nxt, n, 0);
      }
      dma_range<S>(rx, xo, ry, yo, base, pend_buf, pend_kb, wave, r * L / NA, (r + 1) * L / NA);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  __builtin_amdgcn_s_setprio(0);
  wait_vmem<0>();
  __syncthreads();
}

// The two-stage form of that loop for fp8 (64-k MFMA steps, 32-byte fragments).  A stage holds
// only two MFMA k-steps here, so the DMA of a stage stays in the last k-step before the handover:
// issued half of it one k-step later, the second half had one k-step to land and the launch lost
// 10%.  A second full fragment
// set does not fit beside the 8-wave tile's accumulators, so only the Y (B operand) fragments are
// double-buffered and the X fragments rotate in place: X fragment i of the next k-step is read as
// soon as the MFMAs of row i are issued, with the rest of the k-step's MFMAs to land in.  In a
// stage's last k-step the MFMAs of row 0 go out before the barrier, covering the wait for the
// stage's last reads.
template <class S>
__device__ inline void tile_kloop_2s_fp8(i32x4 rx, const uint32_t* xo, i32x4 ry,
                                         const uint32_t* yo, int ksteps, char* lds, int wave,
                                         int lane, f32x16 (&acc)[S::FI][S::FJ]) {
  constexpr int NK = S::SEGS / 4;
  static_assert(S::NS == 2 && NK % 2 == 0, "two stages of an even number of k-steps");
  const int wi = wave / S::WJ, wj = wave % S::WJ;
  const int h2 = (lane >> 5) * 2;
  const uint32_t base = lds_addr(lds);
#pragma unroll
  for (int i = 0; i < S::FI; ++i)
#pragma unroll
    for (int j = 0; j < S::FJ; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;
  if (ksteps <= 0) {
    __syncthreads();
    return;
  }
  issue_loads<S, S::XQ>(rx, xo, 0, base, wave);
  issue_loads<S, S::YQ>(ry, yo, 0, base + S::BI * S::BKB, wave);
  wait_vmem<0>();
  __syncthreads();
  {
    const uint32_t kb = ksteps > 1 ? (uint32_t)S::BKB : kOOB;
    dma_range<S>(rx, xo, ry, yo, base, S::STAGE, kb, wave, 0, S::LOADS);
  }
  const int xrow = wi * S::TM * S::BKB, yrow = (S::BI + wj * S::TN) * S::BKB;
  // k-step kk's fragments of the stage at offset st
  auto xfrag = [&](int st, int f, int kk) {
    return frag_fp8<S::BKB>(lds + st + xrow + f * 32 * S::BKB, kk * 4 + h2, lane);
  };
  auto yfrag = [&](int st, int f, int kk) {
    return frag_fp8<S::BKB>(lds + st + yrow + f * 32 * S::BKB, kk * 4 + h2, lane);
  };
  // format 0 = FP8 E4M3 for both operands; E8M0 scale 127 = 2^0 on both
  auto mma = [](const i32x8& x, const i32x8& y, const f32x16& c) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(x, y, c, 0, 0, 0, 127, 0, 127);
  };
  i32x8 a[S::FI], b[2][S::FJ];
#pragma unroll
  for (int f = 0; f < S::FI; ++f) a[f] = xfrag(0, f, 0);
#pragma unroll
  for (int f = 0; f < S::FJ; ++f) b[0][f] = yfrag(0, f, 0);
  for (int kt = 0; kt < ksteps; ++kt) {
    const int cur = (kt & 1) * S::STAGE, nxt = S::STAGE - cur;
    __builtin_amdgcn_s_setprio(0);
#pragma unroll
    for (int kk = 0; kk < NK - 1; ++kk) {
      const int c = kk & 1;
#pragma unroll
      for (int f = 0; f < S::FJ; ++f) b[c ^ 1][f] = yfrag(cur, f, kk + 1);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < S::FI; ++i) {
#pragma unroll
        for (int j = 0; j < S::FJ; ++j) acc[i][j] = mma(a[i], b[c][j], acc[i][j]);
        __builtin_amdgcn_sched_barrier(0);
        a[i] = xfrag(cur, i, kk + 1);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // last k-step of the stage (Y fragments in set 1: NK is even)
#pragma unroll
    for (int j = 0; j < S::FJ; ++j) acc[0][j] = mma(a[0], b[1][j], acc[0][j]);
    __builtin_amdgcn_sched_barrier(0);
    stage_handover<0>();
    // raised issue priority until the next stage starts, as in tile_kloop_bf16 (ag_fc1_f8
    // GEMM-only 359.1-361.1 -> 354.4-355.0 us, one box)
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int f = 0; f < S::FJ; ++f) b[0][f] = yfrag(nxt, f, 0);
    const uint32_t kb = kt + 2 < ksteps ? (uint32_t)(kt + 2) * S::BKB : kOOB;
#pragma unroll
    for (int i = 0; i < S::FI; ++i) {
      if (i > 0) {
#pragma unroll
        for (int j = 0; j < S::FJ; ++j) acc[i][j] = mma(a[i], b[1][j], acc[i][j]);
      }
      __builtin_amdgcn_sched_barrier(0);
      a[i] = xfrag(nxt, i, 0);
      // the DMA of stage kt + 2 into the buffer just read, spread over the rows
      dma_range<S>(rx, xo, ry, yo, base, cur, kb, wave, i * S::LOADS / S::FI,
                   (i + 1) * S::LOADS / S::FI);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  __builtin_amdgcn_s_setprio(0);
  wait_vmem<0>();
  __syncthreads();
}

// The accumulator layout (MB of acc_row / acc_col) of a tile's K loop by default: 16x16 MFMAs for
// bf16 on the tiles with 128-byte rows, 32x32 otherwise.
template <class S, bool FP8>
constexpr int acc_block() {
  return (!FP8 && S::BKB == 128) ? kAcc16 : kAcc32;
}

// Full K loop of one tile.  rx/ry: descriptors of X and Y; xo/yo from tile_offsets; ksteps = K
// bytes / BKB.  Returns with acc = the wave's fp32 sub-tile, in layout MB, and all waves past a
// final barrier (LDS free for the epilogue).  The caller must have passed a barrier since the
// last LDS reads.  bf16 takes a pipelined loop on every tile (16x16 MFMAs for MB = kAcc16, 32x32
// otherwise), fp8 on the two-stage tiles; the plain loop below (barrier at the start of each
// stage, stage_mma per stage) is left for the 4-stage fp8 tile.
template <class S, bool FP8, int MB = acc_block<S, FP8>()>
__device__ inline void tile_kloop(i32x4 rx, const uint32_t* xo, i32x4 ry, const uint32_t* yo,
                                  int ksteps, char* lds, int wave, int lane,
                                  f32x16 (&acc)[S::FI][S::FJ]) {
  static_assert(MB == kAcc32 || (MB == kAcc16 && !FP8 && S::BKB == 128),
                "16x16 MFMAs: the bf16 loop of the 128-byte-row tiles");
  if constexpr (!FP8) {
    NoStageHook none;
    if constexpr (MB == kAcc16) tile_kloop_bf16<S>(rx, xo, ry, yo, ksteps, lds, wave, lane, acc, none);
    else tile_kloop_bf16_32<S>(rx, xo, ry, yo, ksteps, lds, wave, lane, acc, none);
    return;
  } else if constexpr (S::NS == 2) {
    tile_kloop_2s_fp8<S>(rx, xo, ry, yo, ksteps, lds, wave, lane, acc);
    return;
  }
  const int wi = wave / S::WJ, wj = wave % S::WJ;
  const uint32_t base = lds_addr(lds);
#pragma unroll
  for (int i = 0; i < S::FI; ++i)
#pragma unroll
    for (int j = 0; j < S::FJ; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  // prologue: stages 0 .. NS-2
#pragma unroll
  for (int s = 0; s < S::NS - 1; ++s) {
    if (s < ksteps) {
      const uint32_t st = base + (uint32_t)(s * S::STAGE);
      issue_loads<S, S::XQ>(rx, xo, (uint32_t)(s * S::BKB), st, wave);
      issue_loads<S, S::YQ>(ry, yo, (uint32_t)(s * S::BKB), st + S::BI * S::BKB, wave);
    }
  }
  for (int kt = 0; kt < ksteps; ++kt) {
    // stage kt is complete once at most the loads of the stages after it are outstanding
    if (kt + S::NS - 2 < ksteps) wait_vmem<(S::NS - 2) * S::LOADS>();
    else wait_vmem<0>();
    __syncthreads();
    const int nx = kt + S::NS - 1;
    if (nx < ksteps) {
      const uint32_t st = base + (uint32_t)((nx % S::NS) * S::STAGE);
      issue_loads<S, S::XQ>(rx, xo, (uint32_t)nx * S::BKB, st, wave);
      issue_loads<S, S::YQ>(ry, yo, (uint32_t)nx * S::BKB, st + S::BI * S::BKB, wave);
    }
    const char* st = lds + (kt % S::NS) * S::STAGE;
    stage_mma<S, FP8>(st + wi * S::TM * S::BKB, st + (S::BI + wj * S::TN) * S::BKB, lane, acc);
  }
  __syncthreads();
}

// Output coordinates of accumulator element e of 32x32 block (i, j) for this lane, relative to
// the wave's sub-tile origin; each is a lane part plus a part the same for every lane.
//   kAcc32:  row = 32 i + 8 (e / 4) + 4 (lane / 32) + e % 4,  col = 32 j + lane % 32;
//   kAcc16:  block s = e / 4 = 2 bi + bj:  row = 32 i + 16 bi + 4 (lane / 16) + e % 4,
//            col = 32 j + 16 bj + lane % 16;
//   kAcc16S: row = 32 i + 16 bi + 4 bj + 8 (lane / 32) + e % 4,  col = 32 j + lane % 32.
template <int MB>
__host__ __device__ constexpr int acc_row(int i, int e, int lane) {
  if constexpr (MB == kAcc16) return i * 32 + (e >> 3) * 16 + (lane >> 4) * 4 + (e & 3);
  else if constexpr (MB == kAcc16S)
    return i * 32 + (e >> 3) * 16 + ((e >> 2) & 1) * 4 + (lane >> 5) * 8 + (e & 3);
  else return i * 32 + (e >> 2) * 8 + (lane >> 5) * 4 + (e & 3);
}
template <int MB>
__host__ __device__ constexpr int acc_col(int j, int e, int lane) {
  if constexpr (MB == kAcc16) return j * 32 + ((e >> 2) & 1) * 16 + (lane & 15);
  else return j * 32 + (lane & 31);
}

// kAcc16 -> kAcc16S in registers: in each pair of 16x16 blocks side by side (bj = 0, 1) the
// second and fourth 16-lane rows of the left block trade places with the first and third of the
// right one (v_permlane16_swap), so that a lane's element e then sits at 32 consecutive columns
// across lanes 0-31 (and 32-63) instead of 16: one wave instruction on it covers two whole rows of
// 32 floats (two 128-byte lines) instead of four rows of 16.
template <int FI, int FJ>
__device__ inline void acc_swap_rows16(f32x16 (&acc)[FI][FJ]) {
#pragma unroll
  for (int i = 0; i < FI; ++i)
#pragma unroll
    for (int j = 0; j < FJ; ++j)
#pragma unroll
      for (int bi = 0; bi < 2; ++bi)
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) {
          const int l = 8 * bi + e4, r = 8 * bi + 4 + e4;   // blocks (bi, 0) and (bi, 1)
          const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(acc[i][j][l]),
                                                          __float_as_uint(acc[i][j][r]), false,
                                                          false);
          acc[i][j][l] = __uint_as_float(p[0]);
          acc[i][j][r] = __uint_as_float(p[1]);
        }
}


// Epilogue for bf16 output: the accumulators (times `scale`) are rounded to bf16 into an LDS
// tile, then written out row by row with 16-byte stores.  out points at row 0 / column 0 of the
// tile; ld = row stride in elements; rows/cols valid = how much of the tile lies inside the
// output.  Ends with a barrier (LDS free again).
template <class S, int MB>
__device__ inline void store_tile_bf16(const f32x16 (&acc)[S::FI][S::FJ], float scale, char* lds,
                                       __bf16* out, int ld, int rows_valid, int cols_valid,
                                       int wave, int lane) {
  const int wi = wave / S::WJ, wj = wave % S::WJ;
  // Two adjacent columns per LDS write: lanes 2m and 2m + 1 hold adjacent columns of the same
  // rows, so each packs two of its elements (rows r and r + DR of its column) into one bf16 pair,
  // trades that word with its neighbour (DPP quad_perm [1,0,3,2]) and keeps a pair of one row:
  // the even lane row r, the odd lane row r + DR.  DR = 2 (kAcc16, kAcc32) or 4 (kAcc16S) with
  // the layout's row stride LD puts the odd lanes' words 16 banks (mod 32) past the even lanes'
  // and the lane groups of one write in distinct banks.  Half as many LDS writes as one element
  // per write (ag_4k GEMM-only 97.6 -> 97.0 us, chunked 109.5-110.0 -> 108.4-109.2 us, one box;
  // the same bits).
  constexpr int LD = MB == kAcc32 ? S::OUT_LD32 : S::OUT_LD;
  constexpr int P = MB == kAcc16S ? 4 : 2;   // the partner element
  constexpr int DR = acc_row<MB>(0, P, 0) - acc_row<MB>(0, 0, 0);
  const bool odd = lane & 1;
  // v_perm byte selector: odd lane {nb.hi, own.hi}, even lane {own.lo, nb.lo}
  const uint32_t sel = odd ? 0x03020706u : 0x05040100u;
  char* const wb = lds + (wi * S::TM + acc_row<MB>(0, 0, lane) + (odd ? DR : 0)) * LD +
                   ((wj * S::TN + acc_col<MB>(0, 0, lane)) & ~1) * 2;
#pragma unroll
  for (int i = 0; i < S::FI; ++i)
#pragma unroll
    for (int j = 0; j < S::FJ; ++j) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        if (e & P) continue;
        const f32x2 v = {acc[i][j][e] * scale, acc[i][j][e + P] * scale};
        const uint32_t own = __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
        const uint32_t nb = (uint32_t)__builtin_amdgcn_mov_dpp((int)own, 0xB1, 0xF, 0xF, false);
        const int off = (acc_row<MB>(i, e, 0) - acc_row<MB>(0, 0, 0)) * LD +
                        (acc_col<MB>(j, e, 0) - acc_col<MB>(0, 0, 0)) * 2;
        *(uint32_t*)(wb + off) = __builtin_amdgcn_perm(nb, own, sel);
      }
      __builtin_amdgcn_sched_barrier(0);   // one block at a time: bounds the live temporaries
    }
  __syncthreads();
  constexpr int OSEGS = S::BJ / 8;   // 16-byte segments per tile row
  const bool vec = (ld % 8) == 0 && (((uintptr_t)out) & 15u) == 0;
  for (int idx = threadIdx.x; idx < S::BI * OSEGS; idx += S::NT) {
    const int r = idx / OSEGS, sg = idx % OSEGS;
    const int c = sg * 8;
    if (r >= rows_valid || c >= cols_valid) continue;
    const char* src = lds + r * LD + c * 2;
    __bf16* dst = out + (size_t)r * ld + c;
    if (vec && c + 8 <= cols_valid) {
      // non-temporal: written once, never read back here; keeps the operands in L2
      __builtin_nontemporal_store(*(const i32x4*)src, (i32x4*)dst);
    } else {
      for (int e = 0; e < 8 && c + e < cols_valid; ++e) dst[e] = ((const __bf16*)src)[e];
    }
  }
  __syncthreads();
}

// Epilogue for fp8 (OCP E4M3) output.  v = acc * scale is the GEMM's result; the code is
// E4M3(v * scale_d), saturated to +-448 and rounded to nearest even by the hardware convert; the
// codes are staged through LDS and written out 16 bytes at a time.  Returns this thread's
// max |v| (its share of the output's amax).  Ends with a barrier (LDS free again).
template <class S, int MB>
__device__ inline float store_tile_fp8(const f32x16 (&acc)[S::FI][S::FJ], float scale,
                                       float scale_d, char* lds, uint8_t* out, int ld,
                                       int rows_valid, int cols_valid, int wave, int lane) {
  constexpr int LD8 = S::BJ + 16;
  const int wi = wave / S::WJ, wj = wave % S::WJ;
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < S::FI; ++i)
#pragma unroll
    for (int j = 0; j < S::FJ; ++j) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int col = wj * S::TN + acc_col<MB>(j, e, lane);
        const int row = wi * S::TM + acc_row<MB>(i, e, lane);
        const float v = acc[i][j][e] * scale;
        amax = fmaxf(amax, fabsf(v));
        float q = v * scale_d;
        if (!__builtin_isnan(q)) q = fminf(fmaxf(q, -448.0f), 448.0f);
        lds[row * LD8 + col] = (char)(__builtin_amdgcn_cvt_pk_fp8_f32(q, 0.0f, 0, false) & 0xff);
      }
    }
  __syncthreads();
  constexpr int OSEGS = S::BJ / 16;   // 16-byte segments per tile row
  const bool vec = (ld % 16) == 0 && (((uintptr_t)out) & 15u) == 0;
  for (int idx = threadIdx.x; idx < S::BI * OSEGS; idx += S::NT) {
    const int r = idx / OSEGS, sg = idx % OSEGS;
    const int c = sg * 16;
    if (r >= rows_valid || c >= cols_valid) continue;
    const char* src = lds + r * LD8 + c;
    uint8_t* dst = out + (size_t)r * ld + c;
    if (vec && c + 16 <= cols_valid) {
      __builtin_nontemporal_store(*(const i32x4*)src, (i32x4*)dst);
    } else {
      for (int e = 0; e < 16 && c + e < cols_valid; ++e) dst[e] = (uint8_t)src[e];
    }
  }
  __syncthreads();
  return amax;
}

// Max of v over the workgroup's threads; the result is valid in thread 0.  `red` is an LDS array
// of one float per wave.
template <class S>
__device__ inline float block_max(float v, float* red, int wave, int lane) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  if (lane == 0) red[wave] = v;
  __syncthreads();
  float m = 0.0f;
  if (threadIdx.x == 0)
    for (int w = 0; w < S::NW; ++w) m = fmaxf(m, red[w]);
  __syncthreads();
  return m;
}

}  // namespace ringag
