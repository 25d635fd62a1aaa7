// Loading and launching the library's kernels.
//
// The kernels live in one gfx950 code object (device_kernels.hip, built with hipcc --genco) that
// the build embeds into the shared library as a byte array.  load_kernels() loads it with
// hipModuleLoadData on a device the first time a context is created there and keeps the module
// (and the function handles) until the process ends.  The shared library therefore contains no
// compiler-generated registration constructors or destructors: nothing of it runs at process exit,
// when the HIP runtime itself may already be shutting down.
#include <hip/hip_runtime_api.h>

#include <mutex>

#include "kernels.hpp"

// The HIP runtime's extended module launch (declared in hip_ext.h, whose templates need the HIP
// compiler; this file is plain C++).
extern "C" hipError_t hipExtModuleLaunchKernel(hipFunction_t f, uint32_t globalWorkSizeX,
                                               uint32_t globalWorkSizeY, uint32_t globalWorkSizeZ,
                                               uint32_t localWorkSizeX, uint32_t localWorkSizeY,
                                               uint32_t localWorkSizeZ, size_t sharedMemBytes,
                                               hipStream_t hStream, void** kernelParams,
                                               void** extra, hipEvent_t startEvent,
                                               hipEvent_t stopEvent, uint32_t flags);

extern "C" const unsigned char ringag_kernels_co[];

namespace ringag {
namespace {

constexpr int kMaxDevices = 64;
constexpr int kTiles = kNumTiles;

const char* const kAgName[2][2][kTiles] = {   // [fp8 input][fp8 output][tile]
    {{nullptr, "rag_ag_bf16_t128x128", "rag_ag_bf16_t256x128", "rag_ag_bf16_t256x256",
      "rag_ag_bf16_t256x256w8", "rag_ag_bf16_t256x256w8s4", "rag_ag_bf16_t256x192w8"},
     {nullptr, "rag_ag_bf16_o8_t128x128", "rag_ag_bf16_o8_t256x128", "rag_ag_bf16_o8_t256x256",
      "rag_ag_bf16_o8_t256x256w8", "rag_ag_bf16_o8_t256x256w8s4", "rag_ag_bf16_o8_t256x192w8"}},
    {{nullptr, "rag_ag_fp8_t128x128", "rag_ag_fp8_t256x128", "rag_ag_fp8_t256x256",
      "rag_ag_fp8_t256x256w8", "rag_ag_fp8_t256x256w8s4", "rag_ag_fp8_t256x192w8"},
     {nullptr, "rag_ag_fp8_o8_t128x128", "rag_ag_fp8_o8_t256x128", "rag_ag_fp8_o8_t256x256",
      "rag_ag_fp8_o8_t256x256w8", "rag_ag_fp8_o8_t256x256w8s4", "rag_ag_fp8_o8_t256x192w8"}}};
const char* const kAgSlabName[2][kTiles] = {   // [fp8 output][tile], bf16 input
    {nullptr, nullptr, nullptr, nullptr, "rag_ag_bf16_slab_t256x256w8", nullptr,
     "rag_ag_bf16_slab_t256x192w8"},
    {nullptr, nullptr, nullptr, nullptr, "rag_ag_bf16_o8_slab_t256x256w8", nullptr,
     "rag_ag_bf16_o8_slab_t256x192w8"}};
const char* const kRsName[kTiles] = {nullptr, "rag_rs_t128x128", "rag_rs_t256x128",
                                     "rag_rs_t256x256", "rag_rs_t256x256w8",
                                     "rag_rs_t256x256w8s4", "rag_rs_t256x192w8"};

struct DeviceKernels {
  bool loaded = false;
  hipModule_t module = nullptr;
  hipFunction_t ag[2][2][kTiles] = {};
  hipFunction_t ag_slab[2][kTiles] = {};
  hipFunction_t rs[kTiles] = {};
  hipFunction_t arrival = nullptr;
  int* scratch = nullptr;   // device address of the module's scratch array
};

DeviceKernels g_dev[kMaxDevices];
std::mutex g_mu;

bool valid_tile(int tile) { return tile >= 1 && tile < kTiles; }

// With ev_start / ev_stop, the events are recorded by the kernel's own dispatch (the extended
// launch takes the global work size, grid x threads), so their interval is the kernel's duration
// without the queue time of separate event markers.
hipError_t launch(hipFunction_t f, int grid, int threads, hipStream_t s, void* args,
                  hipEvent_t ev_start = nullptr, hipEvent_t ev_stop = nullptr) {
  if (!f) return hipErrorInvalidDeviceFunction;
  void* params[] = {args};
  if (ev_start || ev_stop)
    return hipExtModuleLaunchKernel(f, (uint32_t)grid * (uint32_t)threads, 1, 1, threads, 1, 1,
                                    0, s, params, nullptr, ev_start, ev_stop, 0);
  return hipModuleLaunchKernel(f, grid, 1, 1, threads, 1, 1, 0, s, params, nullptr);
}

hipError_t info(hipFunction_t f, int threads, KernelInfo* out) {
  if (!f) return hipErrorInvalidDeviceFunction;
  int regs = 0, lds = 0, nb = 0;
  hipError_t e = hipFuncGetAttribute(&regs, HIP_FUNC_ATTRIBUTE_NUM_REGS, f);
  if (e == hipSuccess) e = hipFuncGetAttribute(&lds, HIP_FUNC_ATTRIBUTE_SHARED_SIZE_BYTES, f);
  if (e == hipSuccess) e = hipModuleOccupancyMaxActiveBlocksPerMultiprocessor(&nb, f, threads, 0);
  if (e != hipSuccess) return e;
  out->threads = threads;
  out->lds_bytes = lds;
  out->vgprs_per_wave = regs;
  out->max_blocks_per_cu = nb;
  return hipSuccess;
}

}  // namespace

const char* ag_kernel_name(int tile, bool fp8, bool out8, bool slab) {
  if (!valid_tile(tile)) return "";
  if (slab) return (!fp8 && kAgSlabName[out8 ? 1 : 0][tile]) ? kAgSlabName[out8 ? 1 : 0][tile] : "";
  return kAgName[fp8 ? 1 : 0][out8 ? 1 : 0][tile];
}

bool ag_slab_tile(int tile) { return valid_tile(tile) && kAgSlabName[0][tile] != nullptr; }

const char* rs_kernel_name(int tile) { return valid_tile(tile) ? kRsName[tile] : ""; }

hipError_t load_kernels(int device) {
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  DeviceKernels& d = g_dev[device];
  if (d.loaded) return hipSuccess;
  hipError_t e = hipSetDevice(device);
  if (e != hipSuccess) return e;
  hipModule_t m = nullptr;
  e = hipModuleLoadData(&m, ringag_kernels_co);
  if (e != hipSuccess) return e;
  for (int fp8 = 0; fp8 < 2; ++fp8)
    for (int o8 = 0; o8 < 2; ++o8)
      for (int t = 1; t < kTiles; ++t)
        if ((e = hipModuleGetFunction(&d.ag[fp8][o8][t], m, kAgName[fp8][o8][t])) != hipSuccess)
          return e;
  for (int o8 = 0; o8 < 2; ++o8)
    for (int t = 1; t < kTiles; ++t)
      if (kAgSlabName[o8][t] &&
          (e = hipModuleGetFunction(&d.ag_slab[o8][t], m, kAgSlabName[o8][t])) != hipSuccess)
        return e;
  for (int t = 1; t < kTiles; ++t)
    if ((e = hipModuleGetFunction(&d.rs[t], m, kRsName[t])) != hipSuccess) return e;
  if ((e = hipModuleGetFunction(&d.arrival, m, "rag_arrival")) != hipSuccess) return e;
  // the fixed scratch array: its address on this device (each device's copy of the module has
  // its own), checked for the size the host expects, and cleared once
  hipDeviceptr_t sp = nullptr;
  size_t sbytes = 0;
  if ((e = hipModuleGetGlobal(&sp, &sbytes, m, "scratch")) != hipSuccess) return e;
  if (sp == nullptr || sbytes != sizeof(int) * (size_t)kScratchWords) return hipErrorInvalidSymbol;
  if ((e = hipMemset(sp, 0, sbytes)) != hipSuccess) return e;
  if ((e = hipDeviceSynchronize()) != hipSuccess) return e;
  d.scratch = reinterpret_cast<int*>(sp);
  d.module = m;
  d.loaded = true;
  return hipSuccess;
}

int* device_scratch(int device) {
  if (device < 0 || device >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_mu);
  return g_dev[device].loaded ? g_dev[device].scratch : nullptr;
}

hipError_t launch_ag_gemm(int device, const AgArgs& a, int tile, bool fp8, int grid,
                          hipStream_t s, hipEvent_t ev_start, hipEvent_t ev_stop) {
  const int o8 = a.out_fp8 ? 1 : 0;
  if (device < 0 || device >= kMaxDevices || !g_dev[device].loaded || !valid_tile(tile))
    return hipErrorInvalidValue;
  AgArgs copy = a;
  hipFunction_t f = g_dev[device].ag[fp8 ? 1 : 0][o8][tile];
  if (a.slab.on) f = fp8 ? nullptr : g_dev[device].ag_slab[o8][tile];
  return launch(f, grid, tile_threads(tile), s, &copy, ev_start, ev_stop);
}

hipError_t launch_gemm_rs(int device, const RsArgs& a, int tile, int grid, hipStream_t s,
                          hipEvent_t ev_start, hipEvent_t ev_stop) {
  if (device < 0 || device >= kMaxDevices || !g_dev[device].loaded || !valid_tile(tile))
    return hipErrorInvalidValue;
  RsArgs copy = a;
  return launch(g_dev[device].rs[tile], grid, tile_threads(tile), s, &copy, ev_start, ev_stop);
}

hipError_t launch_arrival(int device, const ArrivalArgs& a, int grid, hipStream_t s) {
  if (device < 0 || device >= kMaxDevices || !g_dev[device].loaded) return hipErrorInvalidValue;
  ArrivalArgs copy = a;
  return launch(g_dev[device].arrival, grid, kArrivalThreads, s, &copy);
}

hipError_t ag_kernel_info(int device, int tile, bool fp8, bool out8, KernelInfo* out) {
  if (device < 0 || device >= kMaxDevices || !g_dev[device].loaded || !valid_tile(tile))
    return hipErrorInvalidValue;
  return info(g_dev[device].ag[fp8 ? 1 : 0][out8 ? 1 : 0][tile], tile_threads(tile), out);
}

hipError_t arrival_kernel_info(int device, KernelInfo* out) {
  if (device < 0 || device >= kMaxDevices || !g_dev[device].loaded) return hipErrorInvalidValue;
  return info(g_dev[device].arrival, kArrivalThreads, out);
}

hipError_t rs_kernel_info(int device, int tile, KernelInfo* out) {
  if (device < 0 || device >= kMaxDevices || !g_dev[device].loaded || !valid_tile(tile))
    return hipErrorInvalidValue;
  return info(g_dev[device].rs[tile], tile_threads(tile), out);
}

}  // namespace ringag
