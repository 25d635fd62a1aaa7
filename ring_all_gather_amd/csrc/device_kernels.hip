// The library's GPU code: every kernel entry point, compiled on its own into one gfx950 code
// object (hipcc --genco).  The host side embeds that object and loads it explicitly per device
// (launch.cpp), so the shared library holds no compiler-generated registration code.
//
// Entry points: rag_ag_<bf16|fp8>[_o8]_<tile> (input dtype; _o8 = E4M3 output),
// rag_ag_bf16[_o8]_slab_<tile> (K-slab gating, 8-wave 2-stage tiles), rag_rs_<tile>, rag_arrival.  Tile names:
//   t128x128, t256x128, t256x256 (4 waves, 2 stages), t256x256w8 (8 waves, 2 stages), t256x256w8s4
//   (8 waves, 4 stages), t256x192w8 (8 waves, 2 stages); see gemm_core.hpp.
#include "arrival_kernel.hpp"
#include "gemm_ag_kernel.hpp"
#include "gemm_rs_kernel.hpp"

using namespace ringag;

// Fixed device scratch of ag_gemm_noalloc, for callers that cannot allocate device memory: the
// ready counters, piece counts and error word that a context otherwise allocates.  Every kernel
// takes its words through a pointer argument; the host looks up this array's device address in
// the module it loaded on each device (hipModuleGetGlobal, once per device) and passes that.
// It is defined with external linkage, at global scope (so its symbol is the plain name), for
// the lookup to find it by name: a file-local array would be a local symbol of the code object.
__device__ __align__(256) int scratch[kScratchWords];

// Waves per SIMD the GEMM+RS kernels are compiled for (the register budget): two where two waves
// fit beside each other anyway (8-wave tiles; 128x128, whose LDS allows two workgroups per CU).
// Without the hint the compiler spreads the epilogue's loop-carried sums over fresh registers and
// halves the 128x128 kernel's occupancy.
template <class S>
constexpr int rs_waves_per_simd() {
  return (S::NW >= 8 || S::LDS <= 80 * 1024) ? 2 : 1;
}

#define RAG_AG_ENTRY(TILE, SHAPE)                                                            \
  extern "C" __global__ void __launch_bounds__(SHAPE::NT) rag_ag_bf16_##TILE(AgArgs a) {    \
    ag_gemm_body<SHAPE, false, false>(a);                                                    \
  }                                                                                          \
  extern "C" __global__ void __launch_bounds__(SHAPE::NT) rag_ag_fp8_##TILE(AgArgs a) {     \
    ag_gemm_body<SHAPE, true, false>(a);                                                     \
  }                                                                                          \
  extern "C" __global__ void __launch_bounds__(SHAPE::NT) rag_ag_bf16_o8_##TILE(AgArgs a) { \
    ag_gemm_body<SHAPE, false, true>(a);                                                     \
  }                                                                                          \
  extern "C" __global__ void __launch_bounds__(SHAPE::NT) rag_ag_fp8_o8_##TILE(AgArgs a) {  \
    ag_gemm_body<SHAPE, true, true>(a);                                                      \
  }                                                                                          \
  extern "C" __global__ void __launch_bounds__(SHAPE::NT, rs_waves_per_simd<SHAPE>())          \
      rag_rs_##TILE(RsArgs a) {                                                              \
    gemm_rs_body<SHAPE>(a);                                                                  \
  }

RAG_AG_ENTRY(t128x128, Tile128x128)
RAG_AG_ENTRY(t256x128, Tile256x128)
RAG_AG_ENTRY(t256x256, Tile256x256)
RAG_AG_ENTRY(t256x256w8, Tile256x256w8)
RAG_AG_ENTRY(t256x256w8s4, Tile256x256w8s4)
RAG_AG_ENTRY(t256x192w8, Tile256x192w8)

// The K-slab-gated AG+GEMM kernels (bf16 input; bf16 or E4M3 output).
#define RAG_AG_SLAB_ENTRY(TILE, SHAPE)                                                         \
  extern "C" __global__ void __launch_bounds__(SHAPE::NT) rag_ag_bf16_slab_##TILE(AgArgs a) {  \
    ag_gemm_body<SHAPE, false, false, true>(a);                                                \
  }                                                                                            \
  extern "C" __global__ void __launch_bounds__(SHAPE::NT)                                      \
      rag_ag_bf16_o8_slab_##TILE(AgArgs a) {                                                   \
    ag_gemm_body<SHAPE, false, true, true>(a);                                                 \
  }

RAG_AG_SLAB_ENTRY(t256x256w8, Tile256x256w8)
RAG_AG_SLAB_ENTRY(t256x192w8, Tile256x192w8)

extern "C" __global__ void __launch_bounds__(kArrivalThreads) rag_arrival(ArrivalArgs a) {
  arrival_body(a);
}
