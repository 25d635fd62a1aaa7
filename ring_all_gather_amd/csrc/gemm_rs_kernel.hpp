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
// Epilogue: the partials are added to the accumulators where they are, in the register layout
// the K loop leaves them in, after one lane swap (kAcc16S, acc_swap_rows16 in gemm_core.hpp).  A
// lane's accumulator element (i, j, e) then sits at row 32 i + 16 (e / 8) + 4 ((e / 4) % 2) +
// 8 (lane / 32) + e % 4 and column 32 j + lane % 32 of the wave's sub-tile, so one load
// instruction of the wave reads two rows of 32 consecutive floats (two whole 128-byte lines), and
// the row offsets are uniform across the wave.  The loads are raw buffer loads: the per-lane
// offset is fixed for the tile, the row offset goes in a scalar register and the column block in
// the immediate field.  A
// thread issues the loads of IB block rows (64 or more floats) before adding them, so a CU has
// 8 waves x 64 lines x 128 bytes in flight rather than what fits in LDS.  fp32 results (send) are
// stored the same way, non-temporal (they stream past L2 instead of displacing the operands); the
// own chunk's bf16 result goes through LDS for 16-byte row stores.
#pragma once

#include "copy_queue.hpp"
#include "gemm_core.hpp"
#include "kernels.hpp"

namespace ringag {

// Cache policy of a raw buffer access with the non-temporal bit set ("nt" on gfx950): for data
// written once and not read back by the kernel, so it does not displace the GEMM's operands in L2.
constexpr int kNonTemporal = 2;

// Bytes from the first element of `rows` rows of stride ld floats (the last one cols long) to the
// end of that region, clamped to a buffer descriptor's 32-bit range; 0 when rows <= 0.
__device__ inline uint32_t region_bytes(int rows, long long ld, int cols) {
  if (rows <= 0) return 0u;
  const long long b = ((long long)(rows - 1) * ld + cols) * 4;
  return b > 0xffffffffll ? 0xffffffffu : (uint32_t)b;
}

// K loop of the GEMM+RS kernels: 16x16 MFMAs where the AG kernels take them (tile_kloop_bf16),
// 32x32 otherwise.
template <class S>
constexpr int rs_loop_block() {
  return S::BKB == 128 ? kAcc16 : kAcc32;
}
// Layout of the accumulators in the epilogue: kAcc16 is swapped to kAcc16S first
// (acc_swap_rows16), since in kAcc16 every load and store of this epilogue would cover four
// 64-byte row pieces instead of two whole 128-byte lines (rs_8k: 173 against 167 us unswapped;
// swapped, 156-157 against 159-160 us for the 32x32 loop, one box).
template <class S>
constexpr int rs_acc_block() {
  return rs_loop_block<S>() == kAcc16 ? kAcc16S : kAcc32;
}

template <class S>
__device__ inline void rs_epilogue(f32x16 (&acc)[S::FI][S::FJ], char* lds, const RsArgs& a, int c,
                                   bool own, int rb, int cb, int wave, int lane) {
  // loads in flight together: IB block rows x EB elements of each 32x32 block (64 floats per
  // lane; 32 for the 4-wave 256x256 tile, whose accumulators take half the registers)
  constexpr int IB = S::FJ * 16 >= 64 ? 1 : 64 / (S::FJ * 16);
  constexpr int EB = S::FJ * 16 >= 64 ? 32 / S::FJ : 16;
  static_assert(S::FI % IB == 0 && 16 % EB == 0, "blocks must divide into load batches");
  constexpr int MB = rs_acc_block<S>();
  const int wi = wave / S::WJ, wj = wave % S::WJ;
  const int r0 = rb * S::BI;                                   // chunk-local first row of the tile
  // the lane's own row and column offsets; element (i, j, e) adds urow(i, e) rows and
  // ucol(j, e) columns, the same for every lane (acc_row / acc_col)
  const int lrow = wi * S::TM + acc_row<MB>(0, 0, lane);
  const int lcol = cb * S::BJ + wj * S::TN + acc_col<MB>(0, 0, lane);
  auto urow = [](int i, int e) { return acc_row<MB>(i, e, 0); };
  auto ucol = [](int j, int e) { return acc_col<MB>(j, e, 0); };
  // what the tile's result gets added to: every peer's partial (own chunk, one-shot), one
  // incoming running sum (ring step), or nothing (another chunk, one-shot)
  const int nadd = a.ring ? (a.partial[c] != nullptr ? 1 : 0) : (own ? a.tp - 1 : 0);
  for (int n = 0; n < nadd; ++n) {
    // one-shot: the n-th peer in increasing rank, skipping this rank; ring: chunk c's sum
    const int p = a.ring ? c : (n < a.self_rank ? n : n + 1);
    const float* part = a.partial[p] + (size_t)r0 * a.ldp;
    // reads past the chunk's last valid element return zero (ragged rows); columns past Mo in
    // earlier rows read the row's padding or the next row, which only feeds elements that are
    // never stored
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)part, 0, (int)region_bytes(a.nc - r0, a.ldp, a.Mo), 0x00020000);
    const int vo = (int)(((long long)lrow * a.ldp + lcol) * 4);
    int rstride = (int)(a.ldp * 4);
    // (opaque here, so the compiler does not hoist the 64 row offsets out of the tile loop and
    // keep them live through the K loop)
    asm volatile("" : "+s"(rstride));
#pragma unroll
    for (int i0 = 0; i0 < S::FI; i0 += IB)
#pragma unroll
      for (int e0 = 0; e0 < 16; e0 += EB) {
        float y[IB][S::FJ][EB];
#pragma unroll
        for (int ii = 0; ii < IB; ++ii)
#pragma unroll
          for (int e = 0; e < EB; ++e) {
            const int r = urow(i0 + ii, e0 + e);
#pragma unroll
            for (int j = 0; j < S::FJ; ++j)
              y[ii][j][e] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
                  rs, vo + 4 * ucol(j, e0 + e), r * rstride, 0));
          }
#pragma unroll
        for (int ii = 0; ii < IB; ++ii)
#pragma unroll
          for (int j = 0; j < S::FJ; ++j)
#pragma unroll
            for (int e = 0; e < EB; ++e) acc[i0 + ii][j][e0 + e] += y[ii][j][e];
      }
  }
  if (own) {
    store_tile_bf16<S, MB>(acc, 1.0f, lds, (__bf16*)a.D + (size_t)r0 * a.Mo + cb * S::BJ, a.Mo,
                           a.nc - r0, a.Mo - cb * S::BJ, wave, lane);
    return;
  }
  // fp32 to send: rows past the chunk fall outside the descriptor and are dropped; columns past
  // Mo are masked per lane
  float* out = a.send + ((size_t)c * a.nc + r0) * a.Mo;
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(out, 0, (int)region_bytes(a.nc - r0, a.Mo, a.Mo),
                                        0x00020000);
  const int vo = (lrow * a.Mo + lcol) * 4;
  int rstride = a.Mo * 4;
  asm volatile("" : "+s"(rstride));
#pragma unroll
  for (int j = 0; j < S::FJ; ++j)
#pragma unroll
    for (int i = 0; i < S::FI; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        if (lcol + ucol(j, e) >= a.Mo) continue;
        const float v = acc[i][j][e];
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), rs, vo + 4 * ucol(j, e),
                                              urow(i, e) * rstride, kNonTemporal);
      }
}

// The tile this workgroup runs in the round [r0, r0 + n) of a grid of `grid` workgroups, for a
// kernel whose chunks have U tiles each.  When every round holds whole chunks, XCD x (workgroups
// w with w % 8 == x) takes the x-th eighth of every chunk in the round, as chunk-local indices in
// a row: a chunk's epilogue traffic (the own chunk's partial reads, another chunk's fp32 stores)
// then goes through all eight XCDs' paths to memory instead of the one or few XCDs that
// round_tile would give it.  Other shapes use round_tile.
__device__ inline int spread_tile(int r0, int n, int grid, int U) {
  if ((grid & 7) != 0 || (U & 7) != 0 || r0 % U != 0 || n % U != 0) return round_tile(r0, n, grid);
  const int w = (int)blockIdx.x, x = w & 7, q = w >> 3;
  const int e = U >> 3;   // tiles of one chunk per XCD
  if (q >= (n / U) * e) return -1;
  return r0 + (q / e) * U + x * e + q % e;
}

// The tile this workgroup runs in round [r0, r0 + n) of the one-shot form when every partial is
// in memory from the start.  A tile of the own chunk reads tp - 1 partials of its block; with the
// own chunk last in ring order those reads all fall in the final round, where they kept half the
// workgroups busy long after the others ran out of tiles (rs_8k: 7 x 32 MiB read by the 128 own
// tiles of the fourth round).  Here each round takes a share of the own chunk in proportion to
// its size, on slots that rotate from round to round (so the own tiles go to different
// workgroups: rs_8k gives each of 128 workgroups one), and fills its other slots with the other
// chunks' tiles in ring order.
// With grid, round and share multiples of 8, XCD x (workgroups w with w % 8 == x) takes its eighth
// of both as contiguous runs, as spread_tile does.  Returns a ring-ordered tile index or -1.
__device__ inline int oneshot_tile(int r0, int n, int grid, int U, int tp) {
  const long long total = (long long)U * tp;
  const int ob = (int)((long long)U * r0 / total);              // own tiles of earlier rounds
  const int oc = (int)((long long)U * (r0 + n) / total) - ob;   // own tiles of this round
  const int nb = r0 - ob;                                       // other tiles of earlier rounds
  const int w = (int)blockIdx.x;
  const bool by_xcd = (grid & 7) == 0 && (n & 7) == 0 && (oc & 7) == 0;
  const int g = by_xcd ? (w & 7) : 0;                           // slot group (XCD)
  const int s = by_xcd ? (w >> 3) : w;                          // slot in the group
  const int S = by_xcd ? n >> 3 : n, O = by_xcd ? oc >> 3 : oc;
  if (s >= S) return -1;
  const int rot = (int)((long long)(r0 / grid) * O % S);
  const int q = (s - rot + S) % S;
  if (q < O) return (tp - 1) * U + ob + g * O + q;
  return nb + g * (S - O) + (q - O);
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
  __shared__ unsigned s_piece;
  if (a.copies) copy_queue_begin(a.cp);

  for (int r0 = 0; r0 < total; r0 += grid) {
    const int n = min(grid, total - r0);
    const int t = (a.ring || a.gated) ? spread_tile(r0, n, grid, U)
                                      : oneshot_tile(r0, n, grid, U, a.tp);
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
    tile_kloop<S, false, rs_loop_block<S>()>(rx, xo, ry, yo, ksteps, lds, wave, lane, acc);
    if constexpr (rs_loop_block<S>() == kAcc16) acc_swap_rows16(acc);
    // gated: wait for what the epilogue reads (the K loop did not need it): chunk c's running sum
    // (ring), or every peer's partial of the own chunk (one-shot).  With in-kernel copies the
    // workgroup copies pieces, in ring order, until each counter it needs is released.
    const bool waits = a.gated && (a.ring ? a.partial[c] != nullptr : own);
    if (waits) {
      int ok = 1;
      for (int k = 0; k < (a.ring ? 1 : a.tp) && ok; ++k) {
        const int idx = a.ring ? c : k;
        if (!a.ring && k == a.self_rank) continue;
        if (a.copies) run_copy_queue<S::NT, 8, false>(a.cp, a.ctr, a.epoch, 0, idx, &s_piece);
        if (threadIdx.x == 0)
          s_ok = wait_ready(a.ctr + idx * kWordStride, a.epoch, a.err, a.spin_limit);
        __syncthreads();
        ok = __builtin_amdgcn_readfirstlane(s_ok);   // uniform: see run_copy_queue
        __syncthreads();
      }
      if (!ok) continue;
    }
    rs_epilogue<S>(acc, lds, a, c, own, rb, cb, wave, lane);
    if (a.copies) {
      run_copy_queue<S::NT, 8, false>(a.cp, a.ctr, a.epoch, 0, -1, &s_piece,
                                      (unsigned)a.copy_quota);
      __syncthreads();   // keeps this thread-0 step and the next tile's apart
    }
  }
  // whatever is left (every piece is taken by a running workgroup, so every count completes)
  if (a.copies) run_copy_queue<S::NT, 8, false>(a.cp, a.ctr, a.epoch, 0, -1, &s_piece);
}

}  // namespace ringag
