// K-slab arrival: the in-GEMM engine's copies of the peers' chunks, waited for one group of K
// stages at a time (the layout and ownership of the pieces are described with SlabPlan).
//
// TransformerEngine issue #1583, C++ listing: the GEMM consumes a chunk once the counter of that
// chunk says it has arrived.  Gating whole chunks serialises one round of tiles behind the copies
// (every tile of a chunk waits for all of it, and the tiles of one round are the whole GEMM when
// the tiles fit the compute units at once).  Here a tile waits only for the K slab its next loads
// read, so every tile starts within the first few microseconds, and the copies of the later slabs
// ride along inside the K loops of all workgroups: one slot of pieces per group of K stages,
// loaded right after one stage handover, stored after the next, flagged after the one after that
// (the handovers of the 2-stage loop wait for every memory operation of the wave, so the loaded
// vectors are in registers and the stores are complete by then).
//
// Coherence.  A piece's stores go through the copying XCD's L2 to the device-wide point (the
// agent-scope write-through policy of the chunk copies), and its flag is stored once every wave's
// stores are complete, as the chunk copies' counts are (copy_queue.hpp).  The flags are read with
// agent-scope loads.  The tile then reads the slab with ordinary loads: they cannot hit a stale
// line, because the tile took an agent-scope acquire (which invalidates the XCD's L2) before its
// first load, and since then no workgroup of this call has read a line of a slab before all of
// that slab's flags were set (lines are 128 bytes and a slab is 512-byte aligned in G, so no line
// holds two slabs).  So the acquire the chunk protocol takes once per tile is not repeated per
// slab, where an L2 invalidate every few stages would cost microseconds each time.
//
// Progress does not depend on which workgroups are resident: a tile that has waited help_ticks
// for a slab copies the slab's missing pieces itself (a piece copied twice is written twice with
// the same bytes), and a workgroup's leftover pieces are copied after its last tile, so every piece
// is copied before the launch ends.
#pragma once

#include <hip/hip_runtime.h>

#include "copy_queue.hpp"
#include "gemm_core.hpp"
#include "kernels.hpp"

namespace ringag {

// Byte offset, within its copy, of the 16-byte vector this thread copies of piece `idx`, or -1
// when that vector lies past the chunk's rows or past the row's K bytes (ragged tails); *c gets
// the copy index.
__device__ inline long long slab_vec_offset(const SlabPlan& s, int n_peer, int idx, uint32_t ldb,
                                            int nc, int* c) {
  const int per_group = n_peer * s.ppc;
  const int g = idx / per_group;
  const int rem = idx - g * per_group;
  *c = rem / s.ppc;
  const int rb = rem - *c * s.ppc;
  const int row = rb * kSlabRows + (int)(threadIdx.x >> 5);
  const uint32_t col = (uint32_t)g * kSlabRowBytes + (threadIdx.x & 31u) * 16u;
  if (row >= nc || col >= ldb) return -1;
  return (long long)row * ldb + col;
}

__device__ inline int slab_flag_index(const SlabPlan& s, int n_peer, int idx) {
  const int per_group = n_peer * s.ppc;
  const int g = idx / per_group;
  const int rem = idx - g * per_group;
  const int c = rem / s.ppc;
  return (c * s.groups + g) * s.ppc + (rem - c * s.ppc);
}

// Load / store this thread's vector of piece idx (an invalid vector loads zeros, stores nothing).
__device__ inline v4i slab_load(const AgArgs& a, int idx, uint32_t ldb) {
  int c;
  const long long off = slab_vec_offset(a.slab, a.cp.n_peer, idx, ldb, a.nc, &c);
  v4i v = {0, 0, 0, 0};
  if (off >= 0) v = *(const v4i*)((const char*)a.cp.src[c] + off);
  return v;
}

__device__ inline void slab_store(const AgArgs& a, int idx, uint32_t ldb, v4i v) {
  int c;
  const long long off = slab_vec_offset(a.slab, a.cp.n_peer, idx, ldb, a.nc, &c);
  const __amdgpu_buffer_rsrc_t d = __builtin_amdgcn_make_buffer_rsrc(
      a.cp.dst[c], 0, (int)((uint32_t)a.nc * ldb), 0x00020000);
  if (off >= 0) __builtin_amdgcn_raw_buffer_store_b128(v, d, (int)off, 0, kCopyStorePolicy);
}

// Flag piece idx as copied by this call (one lane).
__device__ inline void slab_set_flag(const AgArgs& a, int idx) {
  __hip_atomic_store(a.slab.flags + slab_flag_index(a.slab, a.cp.n_peer, idx), a.epoch,
                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Wave 0: the lowest piece row block rb of group g of copy c whose flag is not this call's epoch,
// or -1 when all are (uniform over the wave).
__device__ inline int slab_first_missing(const AgArgs& a, int c, int g) {
  const int* f = a.slab.flags + (c * a.slab.groups + g) * a.slab.ppc;
  const int lane = threadIdx.x & 63;
  for (int b = 0; b < a.slab.ppc; b += 64) {
    const bool miss = b + lane < a.slab.ppc &&
                      __hip_atomic_load(f + b + lane, __ATOMIC_RELAXED,
                                        __HIP_MEMORY_SCOPE_AGENT) != a.epoch;
    const unsigned long long m = __ballot(miss);
    if (m) return b + (int)__builtin_ctzll(m);
  }
  return -1;
}

// Wave 0: wait until group g of copy c is complete, at most help_ticks; true when it is.
__device__ inline bool slab_poll(const AgArgs& a, int c, int g) {
  if (slab_first_missing(a, c, g) < 0) return true;
  const unsigned long long t0 = wall_clock64();
  while (true) {
    __builtin_amdgcn_s_sleep(2);
    if (slab_first_missing(a, c, g) < 0) return true;
    if ((long long)(wall_clock64() - t0) > a.slab.help_ticks) return false;
  }
}

// The whole workgroup: copy the missing pieces of group g of copy c, one at a time, until every
// flag of the group is set.  Each round sets at least one flag, so this ends after ppc rounds.
__device__ inline void slab_help(const AgArgs& a, int c, int g, uint32_t ldb, int* s_word) {
  while (true) {
    if (threadIdx.x < 64) {
      const int rb = slab_first_missing(a, c, g);
      if (threadIdx.x == 0) *s_word = rb;
    }
    __syncthreads();
    const int rb = __builtin_amdgcn_readfirstlane(*s_word);
    __syncthreads();
    if (rb < 0) return;
    const int idx = (g * a.cp.n_peer + c) * a.slab.ppc + rb;
    slab_store(a, idx, ldb, slab_load(a, idx, ldb));
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (threadIdx.x == 0) slab_set_flag(a, idx);
  }
}

// The whole workgroup, outside the K loops: wait for group g of copy c (helping after
// help_ticks), then take the acquire that orders the tile's loads after everything before it.
__device__ inline void slab_gate_tile(const AgArgs& a, int c, uint32_t ldb, int* s_word) {
  if (threadIdx.x < 64) {
    const bool ok = slab_poll(a, c, 0);
    if (threadIdx.x == 0) *s_word = ok ? 1 : 0;
  }
  __syncthreads();
  const int ok = __builtin_amdgcn_readfirstlane(*s_word);
  __syncthreads();
  if (!ok) slab_help(a, c, 0, ldb, s_word);
  if (threadIdx.x == 0) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  __syncthreads();
}

// The whole workgroup, outside the K loops: copy slots [s0, s1) of this workgroup now, eight
// vectors per thread in flight (pieces past the total are skipped), then flag them.
__device__ inline void slab_copy_slots(const AgArgs& a, int s0, int s1, uint32_t ldb) {
  const int w = (int)blockIdx.x, grid = (int)gridDim.x, q = a.slab.q;
  const int n = (s1 - s0) * q;   // pieces of the slots, slot by slot
  auto piece = [&](int k) { return ((s0 + k / q) * grid + w) * q + k % q; };
  for (int k0 = 0; k0 < n; k0 += 8) {
    v4i v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = k0 + u < n ? piece(k0 + u) : a.slab.total;
      if (i < a.slab.total) v[u] = slab_load(a, i, ldb);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = k0 + u < n ? piece(k0 + u) : a.slab.total;
      if (i < a.slab.total) slab_store(a, i, ldb, v[u]);
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (threadIdx.x < 64)
    for (int k = (int)threadIdx.x; k < n; k += 64)
      if (piece(k) < a.slab.total) slab_set_flag(a, piece(k));
}

// The slots a workgroup still owns after slot s: slots s .. (last slot with a piece).
__device__ inline int slab_slots_end(const AgArgs& a) {
  const int w = (int)blockIdx.x, grid = (int)gridDim.x, q = a.slab.q;
  // smallest s with (s * grid + w) * q >= total
  const int per = grid * q;
  const int need = a.slab.total - w * q;
  return need <= 0 ? 0 : (need + per - 1) / per;
}

// Stage hook of the bf16 K loop (tile_kloop_bf16) for a tile under K-slab gating.  Iteration kt's
// handover completes stage kt + 1; right after it the loop starts the loads of stage kt + 2.
// Cycle phases, counted from the iterations kt = 2 mod 4 (where stage kt + 2 opens a group):
//   phase 0: gate the group of stage kt + 2 (wave 0 checks the flags before the barrier; after
//            it, the workgroup helps if the wait gave up), then load this workgroup's next slot
//            into the LDS staging area with the DMA path the tile's own loads use (no registers
//            held);
//   phase 1: store it from there;  phase 2: flag it.
// A cycle starts only where all three phases fall inside the loop (kt + 2 < ksteps).  The gate's
// flags are loaded one stage ahead (right after the handover of phase 3), so that the check finds
// them in registers: an agent-scope load goes to memory, and waiting for it right before the
// barrier would hold up the whole workgroup at every gate.
struct SlabHook {
  const AgArgs& a;
  const int c;            // copy index of the tile's chunk, or -1 (the own chunk: nothing to wait)
  const int ksteps;
  const uint32_t ldb;
  int* const s_word;
  char* const stage;      // LDS staging, kSlabMaxQ pieces of kSlabThreads 16-byte vectors
  int& slot;              // the workgroup's next slot
  int cur = -1;           // first piece of the slot in flight, or -1
  int ahead = 0;          // wave 0: the flag of row block `lane` of the next gate's group, loaded
                          // one stage ahead (row blocks past the first 64 are checked at the gate)

  __device__ bool gate_at(int kt) const {
    return c >= 0 && ((kt + 2) & 3) == 0 && kt + 2 < ksteps;
  }
  __device__ void pre(int kt) {
    if (!gate_at(kt)) return;
    if (threadIdx.x < 64) {
      const int g = (kt + 2) / kSlabStages;
      const int lane = threadIdx.x;
      bool ok = a.slab.ppc <= 64 && __ballot(lane < a.slab.ppc && ahead != a.epoch) == 0;
      if (!ok) ok = slab_poll(a, c, g);
      if (threadIdx.x == 0) *s_word = ok ? 1 : 0;
    }
  }
  __device__ void post(int kt) {
    if (gate_at(kt + 1) && threadIdx.x < 64 && (int)threadIdx.x < a.slab.ppc) {
      const int g = (kt + 3) / kSlabStages;
      ahead = __hip_atomic_load(a.slab.flags + (c * a.slab.groups + g) * a.slab.ppc + threadIdx.x,
                                __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (gate_at(kt) && !__builtin_amdgcn_readfirstlane(*s_word)) {
      __syncthreads();   // every wave has read the word before slab_help writes it
      slab_help(a, c, (kt + 2) / kSlabStages, ldb, s_word);
    }
    if (kt < 2) return;
    const int ph = (kt - 2) & 3;
    const int q = a.slab.q;
    if (ph == 0) {
      cur = -1;
      if (kt + 2 < ksteps) {
        const int i0 = (slot * (int)gridDim.x + (int)blockIdx.x) * q;
        ++slot;
        if (i0 < a.slab.total) {
          cur = i0;
          // (wave-uniform values in scalar registers: the DMA takes its LDS address in m0 and
          // its descriptor in scalar registers)
          const uint32_t base =
              __builtin_amdgcn_readfirstlane(lds_addr(stage) + (threadIdx.x >> 6) * 1024u);
#pragma unroll
          for (int k = 0; k < kSlabMaxQ; ++k) {
            if (k >= q || i0 + k >= a.slab.total) break;
            int cc;
            const long long off =
                slab_vec_offset(a.slab, a.cp.n_peer, i0 + k, ldb, a.nc, &cc);
            const int cu = __builtin_amdgcn_readfirstlane(cc);
            dma16(make_rsrc(a.cp.src[cu], (uint32_t)a.nc * ldb), base + k * 8192u,
                  off >= 0 ? (uint32_t)off : kOOB);
          }
        }
      }
    } else if (ph == 1 && cur >= 0) {
#pragma unroll
      for (int k = 0; k < kSlabMaxQ; ++k) {
        if (k >= q || cur + k >= a.slab.total) break;
        const v4i v = *(const v4i*)(stage + k * 8192 + threadIdx.x * 16);
        slab_store(a, cur + k, ldb, v);
      }
    } else if (ph == 2 && cur >= 0) {
      if ((int)threadIdx.x < q && cur + (int)threadIdx.x < a.slab.total)
        slab_set_flag(a, cur + (int)threadIdx.x);
      cur = -1;
    }
  }
};

}  // namespace ringag
