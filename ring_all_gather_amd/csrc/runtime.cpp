// Host runtime of libringag.so: the C ABI declared in include/ringag.h.
//
// It owns the per-context resources (side stream, fork/join events, ready counters, piece counts, error
// word, epoch, cached gather and staging buffers), validates every argument before enqueueing
// anything, and orders the work of one call:
//
//   caller stream:  [record fork] ...................... GEMM (tiles wait on counters) [wait join]
//   side stream:        [wait fork] arrivals: copy chunk r_1, bump ctr[r_1]; copy r_2, bump ... [record join]
//
// The arrivals are enqueued before the GEMM (nvFuser PR #3392, experiment: posting communication
// before compute gave near-complete overlap), and the side stream is joined back into the caller's
// stream before the call returns (TransformerEngine issue #1583, C++ listing: communication
// streams fork from and join the main stream through events).  Counters are compared with a
// per-call epoch instead of being reset by a kernel, so a late producer of one call can never be
// mistaken for the next call's.
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cstdarg>
#include <mutex>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "ringag.h"
#include "kernels.hpp"

using namespace ringag;

namespace {

// Trivially destructible, so nothing of it runs at thread or process exit.
thread_local char g_last_error[1024];

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
  va_end(ap);
  return code;
}

#define HIPCHK(call)                                                                   \
  do {                                                                                 \
    hipError_t e_ = (call);                                                            \
    if (e_ != hipSuccess)                                                              \
      return fail(RAG_EHIP, "%s failed: %s (%s:%d)", #call, hipGetErrorString(e_),     \
                  __FILE__, __LINE__);                                                 \
  } while (0)

constexpr long long kMaxOperandBytes = 0x7fffffffLL;   // buffer descriptors address < 2 GiB
constexpr int kMaxRsRow = 1 << 20;   // GEMM+RS: floats per row of send and the partials, at most
constexpr int kTimingSlots = 4096;

bool debug_enabled() {
  const char* v = getenv("RAG_DEBUG");
  return v && v[0] && v[0] != '0';
}

}  // namespace

// One set of the device words a call uses, with the host-side state that goes with them: a
// context's own allocation, or (ag_gemm_noalloc) the library's fixed scratch array of a device.
// Layout, kWordStride ints apart: ctr[kMaxTp] (ready counters; a context allocates max_tp) |
// copy-complete counter | piece counts [2 sets][grab, done][kArrSlots] | error word.
struct Words {
  int* ctr = nullptr;
  unsigned* arr = nullptr;
  int* err = nullptr;
  int epoch = 0;
  unsigned arr_seq = 0;   // copying launches so far (selects the set of grab/done counts)
};

struct rag_ctx {
  int device = 0;
  int max_tp = 0;
  hipStream_t side = nullptr;
  hipEvent_t ev_fork = nullptr, ev_join = nullptr;
  hipEvent_t ev_ag = nullptr;          // linear_allreduce: end of the side stream's copies
  // After a copy kernel on the side stream: ev_side marks its end, and the next launch that runs
  // copies on a caller's stream waits for it first (see join_side_copies)
  hipEvent_t ev_side = nullptr;
  bool side_pending = false;
  // SDMA copies may spread over the side stream and up to two more (RAG_OPT_SDMA_STREAMS)
  hipStream_t sdma[2] = {nullptr, nullptr};
  hipEvent_t ev_sdma[2] = {nullptr, nullptr};
  int sdma_streams = 1;
  int comm_cus = 0;      // > 0: the side stream runs only on these compute units (RAG_OPT_COMM_CUS)
  std::vector<hipEvent_t> ev_chunk;   // split form: chunk j copied (created on first use)
  int* words = nullptr;   // the context's device words (hipMalloc at creation), see Words
  Words w;
  void* gbuf = nullptr;
  size_t gbuf_bytes = 0;
  void* stage = nullptr;
  size_t stage_bytes = 0;
  void* rsbuf = nullptr;        // receive buffer of the reduce-scatter's arrivals
  size_t rsbuf_bytes = 0;
  int* slab_flags = nullptr;    // K-slab gating: per-piece epochs (zeroed when allocated)
  size_t slab_flags_bytes = 0;
  int num_cus = 0;
  long long wall_khz = 100000;
  // options
  int copy_engine = RAG_COPY_IN_GEMM;
  int comm_wgs = 128;
  long long spin_us = 2000000;
  long long delay_us = 0;
  unsigned withhold = 0;
  int tile = RAG_TILE_AUTO;
  bool timing = false;
  int wgs_per_cu = 0;
  int copy_priority = 1;
  int gemm_copy_wgs = 0;
  int ag_gate = RAG_GATE_CHUNK;
  // K-slab gating: how long a tile waits for a slab before it copies the slab's missing pieces
  // itself (normally every slab is there long before a tile needs it)
  long long slab_help_us = 20;
  unsigned long long trace_buf = 0;
  long long trace_bytes = 0;
  std::vector<hipEvent_t> t_start, t_stop;
  int n_timed = 0;
  // occupancy cache: [tile][fp8]
  KernelInfo ag_info[kNumTiles][2][2] = {};   // [tile][fp8 input][fp8 output]
  bool ag_info_ok[kNumTiles][2][2] = {};
  KernelInfo rs_info[kNumTiles] = {};
  bool rs_info_ok[kNumTiles] = {};
  KernelInfo arr_info = {};
  bool arr_info_ok = false;
};

namespace {

int ensure_buffer(void** p, size_t* have, size_t need, const char* what) {
  if (*have >= need) return RAG_OK;
  if (*p) {
    hipError_t e = hipFree(*p);
    if (e != hipSuccess) return fail(RAG_EHIP, "hipFree(%s) failed: %s", what, hipGetErrorString(e));
    *p = nullptr;
    *have = 0;
  }
  hipError_t e = hipMalloc(p, need);
  if (e != hipSuccess) {
    *p = nullptr;
    (void)hipGetLastError();
    return fail(RAG_ENOMEM, "cannot allocate the %s (%zu bytes): %s", what, need,
                hipGetErrorString(e));
  }
  *have = need;
  return RAG_OK;
}

// True when p is device memory of `device` (hipMalloc'd, or managed).  Host pointers, pointers
// of another device and unknown addresses are rejected before anything reaches a kernel.
bool on_device(const void* p, int device) {
  hipPointerAttribute_t at;
  if (hipPointerGetAttributes(&at, p) != hipSuccess) {
    (void)hipGetLastError();
    return false;
  }
  return (at.type == hipMemoryTypeDevice || at.type == hipMemoryTypeManaged) && at.device == device;
}

bool misaligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || !na || !nb) return false;
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

// A copy kernel was just enqueued on the side stream.  A launch that runs copies clears the other
// set of piece counts for the next call (copy_queue_begin), and the side stream's kernel may still
// be running, or not yet have started, when the caller's stream moves on: its GEMM waits for the
// copies' counters only, and workgroups that found the queue empty still add to the grab count on
// their way out.  So the next launch that runs copies on a caller's stream waits for the side
// stream's kernel to end first (join_side_copies); launches on the side stream itself are ordered
// by the stream.
int note_side_copies(rag_ctx* c) {
  HIPCHK(hipEventRecord(c->ev_side, c->side));
  c->side_pending = true;
  return RAG_OK;
}

int join_side_copies(rag_ctx* c, hipStream_t stream) {
  if (!c->side_pending) return RAG_OK;
  HIPCHK(hipStreamWaitEvent(stream, c->ev_side, 0));
  c->side_pending = false;
  return RAG_OK;
}

// The fixed scratch array's words of each device (ag_gemm_noalloc), set up by the first
// rag_create on that device.  Shared by every context on the device.
constexpr int kMaxScratchDevices = 64;
static_assert(sizeof(int) * kScratchWords == RAG_SCRATCH_BYTES, "the header states the size");
Words g_scratch_words[kMaxScratchDevices];
std::mutex g_scratch_mu;

int setup_scratch_words(int device) {
  if (device >= kMaxScratchDevices)
    return fail(RAG_EINVAL, "rag_create: device %d is beyond the %d devices the fixed scratch "
                "covers", device, kMaxScratchDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  Words& W = g_scratch_words[device];
  if (W.ctr) return RAG_OK;
  int* base = device_scratch(device);
  if (!base)
    return fail(RAG_EHIP, "rag_create: the fixed scratch array of device %d was not found in "
                "the loaded kernels", device);
  W.ctr = base;
  W.arr = reinterpret_cast<unsigned*>(base + (size_t)(kMaxTp + 1) * kWordStride);
  W.err = base + (size_t)(kMaxTp + 1 + 4 * kArrSlots) * kWordStride;
  return RAG_OK;
}

int next_epoch(Words& W) {
  W.epoch = (W.epoch == 0x7fffffff) ? 1 : W.epoch + 1;
  return W.epoch;
}

// The set of piece counts the next copying launch on W uses, and the other set, which that
// launch clears for the call after it.
void use_count_set(const Words& W, CopyPlan& cp) {
  const unsigned set = W.arr_seq & 1u;
  cp.grab = W.arr + (size_t)set * 2 * kArrSlots * kWordStride;
  cp.done = cp.grab + (size_t)kArrSlots * kWordStride;
  cp.clear_next = W.arr + (size_t)(set ^ 1u) * 2 * kArrSlots * kWordStride;
}

// The largest tile that still gives every compute unit a tile: bigger tiles re-read less from
// L2 per flop, but a grid with idle compute units loses more than that.  Between the two 8-wave
// sizes, 256x256 and 256x192, the one whose persistent rounds leave the compute units less to do
// in all (rounds x tile area, the 256x192 tile's area weighted 1.1 for its higher LDS and operand
// traffic per flop): 256x192 where it fills whole rounds and 256x256 would leave a partial one
// (8 chunks of 1024 rows by 3072 columns: 512 tiles in 2 rounds against 384 in 1.5).
int choose_ag_tile(const rag_ctx* c, int nc, int M, int tp) {
  if (c->tile != RAG_TILE_AUTO) return c->tile;
  auto tiles = [&](int bi, int bj) {
    return (long long)((nc + bi - 1) / bi) * ((M + bj - 1) / bj) * tp;
  };
  if (tiles(256, 256) >= c->num_cus) {
    auto rounds = [&](long long t) { return (t + c->num_cus - 1) / c->num_cus; };
    const double cost256 = (double)rounds(tiles(256, 256)) * 256 * 256;
    const double cost192 = (double)rounds(tiles(256, 192)) * 256 * 192 * 1.1;
    return cost192 < cost256 ? kTile256x192w8 : kTile256x256w8;
  }
  if (tiles(256, 128) >= c->num_cus) return kTile256x128;
  return kTile128x128;
}

// The engines whose copies run inside the GEMM launch (GEMM+RS calls treat all three alike).
bool in_gemm_engine(int e) {
  return e == RAG_COPY_IN_GEMM || e == RAG_COPY_IN_GEMM_ASSIST || e == RAG_COPY_IN_GEMM_SDMA;
}

const char* engine_name(int e) {
  return e == RAG_COPY_SDMA ? "sdma" : e == RAG_COPY_IN_GEMM ? "in-gemm"
         : e == RAG_COPY_IN_GEMM_ASSIST ? "in-gemm+assist"
         : e == RAG_COPY_IN_GEMM_SDMA ? "in-gemm+sdma" : "kernel";
}

// Persistent grid: every workgroup resident at once (so none waits for a slot while others spin
// on counters), a multiple of 8 so that tile t always runs on XCD t % 8.
int persistent_grid(int total_tiles, int num_cus, int blocks_per_cu) {
  int cap = num_cus * std::max(1, blocks_per_cu);
  int g = std::min(total_tiles, cap);
  if (g >= 8) g -= g % 8;
  return std::max(1, g);
}

// Registers per lane to leave for the HIP runtime's stream write-value kernel: hipStreamWriteValue32
// runs as a small kernel on the compute units (it shows in kernel traces), and the SDMA engine
// releases the counters with it.  Measured bounds: a GEMM+RS grid that left 16 registers per lane
// on every SIMD kept it from running (every gated wait ran out its limit), one that left 32 (the
// bf16 256x256 8-wave AG kernel, 240 registers at two waves per SIMD) did not.
constexpr int kStreamOpVgprs = 32;

// Compute units kept free of GEMM workgroups while a kernel that the GEMM waits for runs beside
// it: the copy kernel on the side stream, or the runtime's write-value kernel that releases the
// counters of SDMA copies.  A GEMM workgroup whose tiles wait for them must never fill every
// compute unit so completely that none of their waves can be placed: then, if the GEMM's
// persistent grid is dispatched first, its waiting tiles spin until the limit while the copies or
// the counter writes cannot start (seen with SDMA and the fp8 256x256 8-wave kernel, 254 registers
// at two waves per SIMD: every wait ran out its limit).  Those kernels need few bytes of LDS and
// `room_vgprs` registers per lane; a GEMM that leaves less than that on a SIMD (its resident waves
// times their registers, of the 512 per lane) gets 8 compute units, one per XCD, left out of its
// grid.  room_vgprs = 0: nothing runs beside it.
int reserved_cus(const KernelInfo& g, int room_vgprs) {
  if (room_vgprs <= 0) return 0;
  const int waves_per_simd = std::max(1, g.max_blocks_per_cu * (g.threads / 64) / 4);
  const int regs = (g.vgprs_per_wave + 7) / 8 * 8;
  return waves_per_simd * regs > 512 - room_vgprs ? 8 : 0;
}

// Registers per lane of one copy-kernel wave, rounded up to the allocation granule of 8.
int copy_wave_vgprs(rag_ctx* c, int* out) {
  if (!c->arr_info_ok) {
    HIPCHK(arrival_kernel_info(c->device, &c->arr_info));
    c->arr_info_ok = true;
  }
  *out = (c->arr_info.vgprs_per_wave + 7) / 8 * 8;
  return RAG_OK;
}

int ag_info(rag_ctx* c, int tile, bool fp8, bool out8, const KernelInfo** out) {
  if (!c->ag_info_ok[tile][fp8][out8]) {
    HIPCHK(ag_kernel_info(c->device, tile, fp8, out8, &c->ag_info[tile][fp8][out8]));
    c->ag_info_ok[tile][fp8][out8] = true;
  }
  *out = &c->ag_info[tile][fp8][out8];
  return RAG_OK;
}

// The tile an AG+GEMM launch uses: choose_ag_tile's, except that with the automatic choice and a
// kernel the GEMM waits for running beside it (room_vgprs > 0), an 8-wave 256x256 kernel that
// would need compute units kept free (above) gives way to the 4-stage 8-wave kernel of the same
// tile size if that one leaves room: the kernel beside then runs on every compute unit.
int ag_launch_tile(rag_ctx* c, int nc, int M, int tp, bool fp8, bool out8, int room_vgprs,
                   int* tile) {
  *tile = choose_ag_tile(c, nc, M, tp);
  if (room_vgprs <= 0 || c->tile != RAG_TILE_AUTO || *tile != kTile256x256w8) return RAG_OK;
  const KernelInfo *w8 = nullptr, *s4 = nullptr;
  int rc = ag_info(c, kTile256x256w8, fp8, out8, &w8);
  if (!rc) rc = ag_info(c, kTile256x256w8s4, fp8, out8, &s4);
  if (rc) return rc;
  if (reserved_cus(*w8, room_vgprs) > 0 && reserved_cus(*s4, room_vgprs) == 0)
    *tile = kTile256x256w8s4;
  return RAG_OK;
}

// How one AG+GEMM call runs (everything but the split form): the copy engine's parts, the tile,
// the persistent grid, and the late queue of the assisting copy kernel.
struct AgPlan {
  bool gemm_copies = false;   // the GEMM launch's workgroups copy
  bool side_kernel = false;   // a copy kernel runs on the side stream
  bool sdma = false;          // SDMA copies on the side streams
  bool assist = false;
  bool hybrid = false;        // in-GEMM copies of the early chunks, SDMA for the late ones
  int room_vgprs = 0;         // registers per lane the GEMM leaves for what it waits for
  int tile = 0, tiles_i = 0, tiles_j = 0, grid = 0;
  int late = 0;               // peers in the late queue (assisting kernel or SDMA)
  SlabPlan slab = {};         // slab.on: K-slab gating (the in-GEMM copies of the peers' chunks)
};

// K-slab gating of a call (SlabPlan), when asked for and where it applies: the in-GEMM engine
// copying the peers' chunks for a bf16 GEMM on an 8-wave 2-stage tile, no test hook that holds copies back, the
// context's own device words, G 128-byte aligned (so that no 128-byte line holds two slabs), and
// at most kSlabMaxQ pieces of each group per workgroup.  Slots hold q pieces: one piece per
// workgroup and group of K when a group has at most `grid` pieces, else two.  `pre`: slots
// copied before the first tile, enough that group 0 is complete and that every later group g is
// flagged two stages before a tile reaches its gate (slot S(g) holds g's last piece; the K loop
// flags slot pre + i at stage 4 i + 4 and gates group g at stage 4 g - 2).
void plan_slab(const rag_ctx* c, int nc, int K, int tp, bool fp8, bool copy_only, bool ctx_words,
               const void* G, AgPlan* p) {
  SlabPlan& s = p->slab;
  s = SlabPlan{};
  if (c->ag_gate != RAG_GATE_SLAB || !p->gemm_copies || p->assist || fp8 || copy_only ||
      !ctx_words || tp < 2 || !ag_slab_tile(p->tile) || c->delay_us > 0 || c->withhold != 0 ||
      (reinterpret_cast<uintptr_t>(G) & 127u) != 0)
    return;
  const long long ldb = 2LL * K;
  const int groups = (int)((ldb + kSlabRowBytes - 1) / kSlabRowBytes);
  const int ppc = (nc + kSlabRows - 1) / kSlabRows;
  const long long per_group = (long long)(tp - 1) * ppc;
  const int q = per_group <= p->grid ? 1 : 2;
  if (per_group > (long long)kSlabMaxQ * p->grid) return;
  const long long per_slot = (long long)p->grid * q;
  auto last_slot = [&](long long g) { return ((g + 1) * per_group + per_slot - 1) / per_slot - 1; };
  long long pre = last_slot(0) + 1;
  for (long long g = 1; g < groups; ++g) pre = std::max(pre, last_slot(g) - g + 2);
  const long long total = per_group * groups;
  if (pre > 4 || total > (1LL << 30)) return;
  s.on = 1;
  s.groups = groups;
  s.ppc = ppc;
  s.q = q;
  s.pre = (int)pre;
  s.total = (int)total;
  s.help_ticks = c->slab_help_us * c->wall_khz / 1000;
}

int plan_ag(rag_ctx* c, int nc, int M, int tp, bool fp8, bool out8, bool no_copy, AgPlan* p) {
  const int engine = c->copy_engine;
  p->assist = !no_copy && engine == RAG_COPY_IN_GEMM_ASSIST;
  p->hybrid = !no_copy && engine == RAG_COPY_IN_GEMM_SDMA;
  p->gemm_copies = !no_copy && (engine == RAG_COPY_IN_GEMM || p->assist || p->hybrid);
  p->side_kernel = !no_copy && (engine == RAG_COPY_KERNEL || p->assist);
  p->sdma = !no_copy && (engine == RAG_COPY_SDMA || p->hybrid);
  int copy_vgprs = 0;
  if (p->side_kernel) {
    const int rc = copy_wave_vgprs(c, &copy_vgprs);
    if (rc) return rc;
  }
  // With the assisting copy kernel, or SDMA for the late chunks: the chunks at ring positions the
  // first round of the grid does not reach (P = ceil(grid / U) and on) are the late queue, which
  // the copy kernel or SDMA takes beside the first round; the GEMM's waiting workgroups copy the
  // early ones.  Without late chunks (one round holds every chunk) nothing runs beside the GEMM
  // and the call is the in-GEMM one.  The first pass plans the GEMM with nothing beside it; when
  // there are late chunks the second plans it with the room the side kernel needs (which may
  // change the tile, and so the late queue).
  for (int pass = 0; pass < 2; ++pass) {
    const bool beside = p->side_kernel && !(p->assist && pass == 0);
    const bool sdma_beside = p->sdma && !(p->hybrid && pass == 0);
    p->room_vgprs = beside ? copy_vgprs : sdma_beside ? kStreamOpVgprs : 0;
    int rc = ag_launch_tile(c, nc, M, tp, fp8, out8, p->room_vgprs, &p->tile);
    if (rc) return rc;
    const KernelInfo* info = nullptr;
    rc = ag_info(c, p->tile, fp8, out8, &info);
    if (rc) return rc;
    int bi, bj;
    tile_dims(p->tile, &bi, &bj);
    p->tiles_i = (nc + bi - 1) / bi;
    p->tiles_j = (M + bj - 1) / bj;
    int bpc = info->max_blocks_per_cu;
    if (c->wgs_per_cu > 0) bpc = std::min(bpc, c->wgs_per_cu);
    p->grid = persistent_grid(p->tiles_i * p->tiles_j * tp,
                              c->num_cus - reserved_cus(*info, p->room_vgprs), bpc);
    if (!p->assist && !p->hybrid) break;
    const int U = p->tiles_i * p->tiles_j;
    p->late = std::max(0, tp - std::max(1, (p->grid + U - 1) / U));
    if (p->late == 0) {
      p->side_kernel = false;
      p->sdma = false;
      break;
    }
  }
  return RAG_OK;
}

int choose_rs_tile(const rag_ctx* c, int nc, int Mo, int tp) {
  return choose_ag_tile(c, nc, Mo, tp);   // same GEMM core and the same trade-off
}

int record_timing_start(rag_ctx* c, hipStream_t s, bool* recorded) {
  *recorded = false;
  if (!c->timing || c->n_timed >= (int)c->t_start.size()) return RAG_OK;
  HIPCHK(hipEventRecord(c->t_start[c->n_timed], s));
  *recorded = true;
  return RAG_OK;
}

int record_timing_stop(rag_ctx* c, hipStream_t s, bool recorded) {
  if (!recorded) return RAG_OK;
  HIPCHK(hipEventRecord(c->t_stop[c->n_timed], s));
  c->n_timed++;
  return RAG_OK;
}

// For a call that is one GEMM launch: the next timing slot's events, which the launch itself
// records around the kernel (both null when timing is off or the slots are used up).  The slot
// counts as used once the launch has succeeded (launch_timed).
void launch_timing_events(rag_ctx* c, hipEvent_t* start, hipEvent_t* stop) {
  *start = *stop = nullptr;
  if (!c->timing || c->n_timed >= (int)c->t_start.size()) return;
  *start = c->t_start[c->n_timed];
  *stop = c->t_stop[c->n_timed];
}

void launch_timed(rag_ctx* c, hipEvent_t start) {
  if (start) c->n_timed++;
}

}  // namespace

namespace {

// Staged output (RAG_STAGED_OUT): slot j of the staging buffer holds the chunk at ring position j;
// move the slots to D's rank offsets.
int finalize_staged(rag_ctx* c, void* D, int nc, int M, int tp, const int* order, int oesz,
                    hipStream_t stream) {
  const size_t dchunk = (size_t)nc * M * oesz;
  char* st = (char*)c->stage;
  bool rotation = true;   // slot j holds chunk j-1 and slot 0 chunk tp-1
  for (int j = 0; j < tp; ++j)
    if (order[j] != (j + tp - 1) % tp) rotation = false;
  if (rotation) {
    // the listing's two copies: first chunk to the spare slot, then slots 1..tp are D
    HIPCHK(hipMemcpyAsync(st + (size_t)tp * dchunk, st, dchunk, hipMemcpyDeviceToDevice, stream));
    HIPCHK(hipMemcpyAsync(D, st + dchunk, (size_t)tp * dchunk, hipMemcpyDeviceToDevice, stream));
  } else {
    for (int j = 0; j < tp; ++j)
      HIPCHK(hipMemcpyAsync((char*)D + (size_t)order[j] * dchunk, st + (size_t)j * dchunk,
                            dchunk, hipMemcpyDeviceToDevice, stream));
  }
  return RAG_OK;
}

// Split form of AG+GEMM (RAG_PER_CHUNK): the side stream copies the peers' chunks in ring order,
// recording an event after each; the caller's stream launches one GEMM per chunk in ring order,
// each after waiting for its chunk's event.  The GEMM of one chunk is the same kernel with tp = 1
// and no counters.  The own chunk's copy into G (if any) goes last, and the caller's stream waits
// for the side stream's end before the call's later work.
int ag_gemm_split(rag_ctx* c, Words& W, const void* A, int M, int K, const void* const* B,
                  int nc, int tp, int self_rank, char* Gp, bool own_copy, void* D, bool fp8,
                  const float* scale_A, const float* scale_B, bool out8, const float* scale_D, float* amax_D,
                  void* B_copy, bool staged, bool no_copy, bool copy_only, long long chunk_bytes,
                  const int* order, int epoch, hipStream_t stream) {
  if (c->ev_chunk.empty()) {
    c->ev_chunk.resize(c->max_tp, nullptr);
    for (auto& ev : c->ev_chunk) HIPCHK(hipEventCreateWithFlags(&ev, hipEventDisableTiming));
  }
  if (!no_copy) {
    HIPCHK(hipEventRecord(c->ev_fork, stream));
    HIPCHK(hipStreamWaitEvent(c->side, c->ev_fork, 0));
    for (int j = 1; j <= tp + 1; ++j) {   // j == tp: the own chunk into G, j == tp+1: B_copy
      const void* src;
      void* dst;
      if (j < tp) {
        src = B[order[j]];
        dst = Gp + (size_t)order[j] * chunk_bytes;
      } else if (j == tp && own_copy) {
        src = B[self_rank];
        dst = Gp + (size_t)self_rank * chunk_bytes;
      } else if (j == tp + 1 && B_copy) {
        src = B[self_rank];
        dst = B_copy;
      } else {
        continue;
      }
      if (c->copy_engine == RAG_COPY_SDMA) {
        HIPCHK(hipMemcpyAsync(dst, src, (size_t)chunk_bytes, hipMemcpyDeviceToDeviceNoCU,
                              c->side));
      } else {
        ArrivalArgs aa = {};
        aa.cp.src[0] = src;
        aa.cp.dst[0] = dst;
        aa.cp.ctr_index[0] = -1;
        aa.cp.pos[0] = j < tp ? j : 0;
        aa.cp.n_peer = 1;
        aa.cp.n = 1;
        aa.cp.bytes = (unsigned long long)chunk_bytes;
        aa.cp.piece_bytes = (unsigned)kArrivalThreads * 256u;
        aa.cp.pieces = (unsigned)((aa.cp.bytes + aa.cp.piece_bytes - 1) / aa.cp.piece_bytes);
        use_count_set(W, aa.cp);
        aa.cp.delay_ticks = c->delay_us * c->wall_khz / 1000;
        aa.ctr = W.ctr;
        aa.epoch = epoch;
        aa.raise_priority = c->copy_priority;
        HIPCHK(launch_arrival(c->device, aa, c->comm_wgs, c->side));
        W.arr_seq++;
        const int rc = note_side_copies(c);
        if (rc) return rc;
      }
      if (j < tp) HIPCHK(hipEventRecord(c->ev_chunk[j], c->side));
    }
    HIPCHK(hipEventRecord(c->ev_join, c->side));
  }
  if (!copy_only) {
    const int tile = choose_ag_tile(c, nc, M, 1);
    if (!c->ag_info_ok[tile][fp8][out8]) {
      HIPCHK(ag_kernel_info(c->device, tile, fp8, out8, &c->ag_info[tile][fp8][out8]));
      c->ag_info_ok[tile][fp8][out8] = true;
    }
    int bi, bj;
    tile_dims(tile, &bi, &bj);
    AgArgs a = {};
    a.A = A;
    a.M = M;
    a.K = K;
    a.nc = nc;
    a.tp = 1;
    a.ctr_index[0] = -1;
    a.join_index = -1;
    a.ctr = W.ctr;
    a.epoch = epoch;
    a.err = W.err;
    a.spin_limit = c->spin_us * c->wall_khz / 1000;
    a.scale_A = scale_A;
    a.scale_B = scale_B;
    a.tiles_i = (nc + bi - 1) / bi;
    a.tiles_j = (M + bj - 1) / bj;
    a.compute = 1;
    a.copy_stride = 1;
    a.out_fp8 = out8 ? 1 : 0;
    a.scale_D = scale_D;
    a.amax_D = amax_D;
    int bpc = c->ag_info[tile][fp8][out8].max_blocks_per_cu;
    if (c->wgs_per_cu > 0) bpc = std::min(bpc, c->wgs_per_cu);
    const int grid = persistent_grid(a.tiles_i * a.tiles_j, c->num_cus, bpc);
    const size_t dchunk = (size_t)nc * M * (out8 ? 1 : 2);
    bool rec = false;
    int rc = record_timing_start(c, stream, &rec);
    if (rc) return rc;
    for (int j = 0; j < tp; ++j) {
      const int r = order[j];
      if (!no_copy && j > 0) HIPCHK(hipStreamWaitEvent(stream, c->ev_chunk[j], 0));
      a.chunk[0] = (j == 0) ? B[self_rank] : (const void*)(Gp + (size_t)r * chunk_bytes);
      a.out[0] = staged ? (void*)((char*)c->stage + (size_t)j * dchunk)
                        : (void*)((char*)D + (size_t)r * dchunk);
      HIPCHK(launch_ag_gemm(c->device, a, tile, fp8, grid, stream));
    }
    rc = record_timing_stop(c, stream, rec);
    if (rc) return rc;
  }
  if (!no_copy) HIPCHK(hipStreamWaitEvent(stream, c->ev_join, 0));
  return RAG_OK;
}

// gemm_rs (ring = false) and gemm_rs_ring (ring = true).  ptrs: by rank, the peers' [T, Mo]
// partials (one-shot), or by chunk, the incoming [nc, Mo] running sums (ring step); ld = their
// row stride.
int rs_call(rag_ctx* c, const char* fn, bool ring, const void* X, int T, int Kl, const void* W,
            int Mo, const float* const* ptrs, long long ld, int tp, int self_rank, float* send,
            void* D, int flags, void* stream_v, bool validate_only = false,
            bool other_copies_beside = false, const CopyPlan* extra_copies = nullptr) {
  if (!c) return fail(RAG_EINVAL, "%s: ctx is NULL", fn);
  if (tp < 1 || tp > c->max_tp)
    return fail(RAG_EINVAL, "%s: tp=%d outside [1, %d] (max_tp of the context)", fn, tp,
                c->max_tp);
  if (self_rank < 0 || self_rank >= tp)
    return fail(RAG_EINVAL, "%s: self_rank=%d outside [0, tp=%d)", fn, self_rank, tp);
  if (T < 1 || Kl < 1 || Mo < 1)
    return fail(RAG_EINVAL, "%s: T=%d, Kl=%d, Mo=%d must all be >= 1", fn, T, Kl, Mo);
  if (T % tp) return fail(RAG_EINVAL, "%s: T=%d is not a multiple of tp=%d", fn, T, tp);
  if (Kl % 64) return fail(RAG_EINVAL, "%s: Kl=%d must be a multiple of 64", fn, Kl);
  if (Mo % 4) return fail(RAG_EINVAL, "%s: Mo=%d must be a multiple of 4", fn, Mo);
  if (flags & ~RAG_RS_ARRIVE) return fail(RAG_EINVAL, "%s: unknown flags 0x%x", fn, flags);
  const bool arrive = (flags & RAG_RS_ARRIVE) != 0;
  if (!X || !W || !D) return fail(RAG_EINVAL, "%s: X, W and D must not be NULL", fn);
  const int nc = T / tp;
  // which entries of ptrs the call reads
  const int start = ((self_rank - 1) % tp + tp) % tp;   // ring: the chain that starts here
  auto used = [&](int i) { return ring ? i != start : i != self_rank; };
  bool any = false;
  for (int i = 0; i < tp; ++i) any = any || used(i);
  if (any && !ptrs) return fail(RAG_EINVAL, "%s: the pointer array must not be NULL", fn);
  const char* ldname = ring ? "ldi" : "ldp";
  if (ld < Mo) return fail(RAG_EINVAL, "%s: %s=%lld must be >= Mo=%d", fn, ldname, ld, Mo);
  // the epilogue addresses a tile's rows with 32-bit offsets
  if (Mo > kMaxRsRow || ld > kMaxRsRow)
    return fail(RAG_EINVAL, "%s: Mo=%d and %s=%lld must be at most %d", fn, Mo, ldname, ld,
                kMaxRsRow);
  if (arrive && ld != Mo)
    return fail(RAG_EINVAL, "%s: RAG_RS_ARRIVE needs %s equal to Mo", fn, ldname);
  if (misaligned(X) || misaligned(W) || misaligned(D) || (send && misaligned(send)))
    return fail(RAG_EINVAL, "%s: X, W, send and D must be 16-byte aligned", fn);
  {
    HIPCHK(hipSetDevice(c->device));
    const void* named[] = {X, W, D, send};
    const char* names[] = {"X", "W", "D", "send"};
    for (int i = 0; i < 4; ++i)
      if (named[i] && !on_device(named[i], c->device))
        return fail(RAG_EINVAL, "%s: %s is not device memory of device %d", fn, names[i],
                    c->device);
  }
  const long long x_bytes = (long long)T * Kl * 2, w_bytes = (long long)Mo * Kl * 2;
  if (x_bytes > kMaxOperandBytes || w_bytes > kMaxOperandBytes)
    return fail(RAG_EINVAL, "%s: X (%lld B) and W (%lld B) must be < 2 GiB", fn, x_bytes,
                w_bytes);
  const long long d_bytes = (long long)nc * Mo * 2;
  const long long send_bytes = (long long)tp * nc * Mo * 4;
  const long long pb = ((long long)((ring ? nc : T) - 1) * ld + Mo) * 4;   // bytes spanned
  for (int i = 0; i < tp; ++i) {
    if (!used(i)) continue;
    if (!ptrs[i]) return fail(RAG_EINVAL, "%s: entry %d of the pointer array is NULL", fn, i);
    if ((reinterpret_cast<uintptr_t>(ptrs[i]) & 3u) != 0)
      return fail(RAG_EINVAL, "%s: entry %d of the pointer array is not 4-byte aligned", fn, i);
    if (!on_device(ptrs[i], c->device))
      return fail(RAG_EINVAL, "%s: entry %d of the pointer array is not device memory of "
                  "device %d", fn, i, c->device);
    if (overlaps(D, d_bytes, ptrs[i], pb) || (send && overlaps(send, send_bytes, ptrs[i], pb)))
      return fail(RAG_EINVAL, "%s: D and send must not overlap entry %d of the pointer array",
                  fn, i);
  }
  if (overlaps(D, d_bytes, X, x_bytes) || overlaps(D, d_bytes, W, w_bytes) ||
      (send && (overlaps(send, send_bytes, X, x_bytes) || overlaps(send, send_bytes, W, w_bytes) ||
                overlaps(send, send_bytes, D, d_bytes))))
    return fail(RAG_EINVAL, "%s: D and send must not overlap X, W or each other", fn);
  if (arrive && c->copy_engine == RAG_COPY_SDMA && c->delay_us > 0)
    return fail(RAG_EINVAL, "%s: the arrival delay hook needs the kernel copy engine", fn);
  if (validate_only) return RAG_OK;

  HIPCHK(hipSetDevice(c->device));
  hipStream_t stream = (hipStream_t)stream_v;
  const long long slot = (long long)nc * Mo;   // floats per receive slot
  if (arrive && any) {
    int rc = ensure_buffer(&c->rsbuf, &c->rsbuf_bytes, (size_t)tp * slot * 4, "receive buffer");
    if (rc) return rc;
  }
  const int epoch = next_epoch(c->w);
  RsArgs a = {};
  a.X = X;
  a.W = W;
  a.ring = ring ? 1 : 0;
  for (int j = 0; j < tp; ++j)
    a.chunk_of[j] = ring ? ((self_rank - 1 - j) % tp + tp) % tp : (self_rank + 1 + j) % tp;
  for (int i = 0; i < tp; ++i) {
    if (!used(i)) continue;
    if (arrive) a.partial[i] = (const float*)c->rsbuf + (size_t)i * slot;
    else a.partial[i] = ring ? ptrs[i] : ptrs[i] + (size_t)self_rank * nc * ld;
  }
  a.ldp = arrive ? Mo : ld;
  a.send = send;
  a.D = D;
  a.T = T;
  a.Kl = Kl;
  a.Mo = Mo;
  a.nc = nc;
  a.tp = tp;
  a.self_rank = self_rank;
  a.gated = arrive && any;
  a.ctr = c->w.ctr;
  a.epoch = epoch;
  a.err = c->w.err;
  a.spin_limit = c->spin_us * c->wall_khz / 1000;

  // Arrivals: copies, in ring order, of what each tile's epilogue reads, releasing one counter per
  // copy; the tiles wait for them on the device.  With the in-GEMM engine the GEMM's own
  // workgroups run them, unless other copies run beside this call (linear_allreduce's gather,
  // whose copy kernel uses the other set of piece counts that a copying launch clears); else the
  // side stream does.
  // extra_copies (linear_allreduce's gather, not gated): copies with nothing waiting for them on
  // the device, run by the same launch
  const bool ig_engine =
      in_gemm_engine(c->copy_engine);
  const bool in_gemm = (a.gated && ig_engine && !other_copies_beside) || extra_copies != nullptr;
  bool join = false;
  if (a.gated) {
    CopyPlan cp = {};
    int n = 0;
    for (int k = 1; k < tp; ++k) {
      // one-shot: peers in arrival order s-1, s-2, ...; ring: chunks in the ring order after the
      // chain that starts here
      const int i = ring ? ((self_rank - 1 - k) % tp + tp) % tp : ((self_rank - k) % tp + tp) % tp;
      cp.src[n] = ring ? (const void*)ptrs[i] : (const void*)(ptrs[i] + (size_t)self_rank * nc * ld);
      cp.dst[n] = (float*)c->rsbuf + (size_t)i * slot;
      cp.ctr_index[n] = i;
      cp.pos[n] = k;
      ++n;
    }
    cp.n_peer = n;
    cp.n = n;
    cp.bytes = (unsigned long long)slot * 4;
    cp.piece_bytes = (unsigned)kArrivalThreads * 256u;
    cp.pieces = (unsigned)((cp.bytes + cp.piece_bytes - 1) / cp.piece_bytes);
    use_count_set(c->w, cp);
    cp.delay_ticks = c->delay_us * c->wall_khz / 1000;
    cp.withhold_mask = c->withhold;
    if (in_gemm) {
      a.copies = 1;
      a.cp = cp;
      c->w.arr_seq++;
    } else {
      HIPCHK(hipEventRecord(c->ev_fork, stream));
      HIPCHK(hipStreamWaitEvent(c->side, c->ev_fork, 0));
      if (c->copy_engine == RAG_COPY_SDMA) {
        for (int k = 0; k < cp.n; ++k) {
          HIPCHK(hipMemcpyAsync(cp.dst[k], cp.src[k], (size_t)cp.bytes, hipMemcpyDeviceToDeviceNoCU,
                                c->side));
          if (!((c->withhold >> cp.pos[k]) & 1u))
            HIPCHK(hipStreamWriteValue32(c->side, c->w.ctr + (size_t)cp.ctr_index[k] * kWordStride,
                                         (uint32_t)epoch, 0));
        }
      } else {
        ArrivalArgs aa = {};
        aa.cp = cp;
        aa.ctr = c->w.ctr;
        aa.epoch = epoch;
        aa.raise_priority = c->copy_priority;
        HIPCHK(launch_arrival(c->device, aa, c->comm_wgs, c->side));
        c->w.arr_seq++;
        const int rc = note_side_copies(c);
        if (rc) return rc;
      }
      // every copy is waited for by some tile, except the ring step's passed-on sums when send is
      // NULL (those tiles are skipped): then the caller's stream waits for the side stream
      join = ring && !send;
      if (join) HIPCHK(hipEventRecord(c->ev_join, c->side));
    }
  }

  if (extra_copies) {
    a.copies = 1;
    a.cp = *extra_copies;
    use_count_set(c->w, a.cp);
    c->w.arr_seq++;
  }
  const bool beside =
      ((a.gated && !in_gemm) || other_copies_beside) && c->copy_engine != RAG_COPY_SDMA;
  int tile = choose_rs_tile(c, nc, Mo, tp);
  for (int t : {tile, (int)kTile256x128, (int)kTile128x128}) {
    if (!c->rs_info_ok[t]) {
      HIPCHK(rs_kernel_info(c->device, t, &c->rs_info[t]));
      c->rs_info_ok[t] = true;
    }
  }
  // Room the GEMM leaves for what runs beside it: the copy kernel's waves, or, with gated SDMA
  // arrivals, the runtime's write-value kernel that releases their counters (see reserved_cus).
  // The automatic choice prefers a tile that leaves every compute unit that room: the copies
  // then spread over the whole GPU instead of 8 CUs.
  int room_vgprs = 0;
  if (a.gated && !in_gemm && c->copy_engine == RAG_COPY_SDMA) {
    room_vgprs = kStreamOpVgprs;
  } else if (beside) {
    const int rc = copy_wave_vgprs(c, &room_vgprs);
    if (rc) return rc;
  }
  if (room_vgprs > 0 && c->tile == RAG_TILE_AUTO &&
      reserved_cus(c->rs_info[tile], room_vgprs) > 0) {
    for (int t : {(int)kTile256x128, (int)kTile128x128})
      if (reserved_cus(c->rs_info[t], room_vgprs) == 0) {
        tile = t;
        break;
      }
  }
  int bi, bj;
  tile_dims(tile, &bi, &bj);
  a.tiles_i = (nc + bi - 1) / bi;
  a.tiles_j = (Mo + bj - 1) / bj;
  const int total = a.tiles_i * a.tiles_j * tp;
  const int grid = persistent_grid(total, c->num_cus - reserved_cus(c->rs_info[tile], room_vgprs),
                                   c->rs_info[tile].max_blocks_per_cu);
  if (in_gemm) {
    // Pieces of (all bytes) / grid rounded up to a power of two from 64 KiB to 1 MiB: a piece
    // costs a take, two barriers, a full wait and an agent-scope release, so at rs_8k (224 MiB)
    // 64 KiB pieces copied at 1.9 TB/s and 1 MiB pieces at well over twice that (896 KiB pieces
    // were 5% slower than 1 MiB, 2 MiB 10%).  After each tile a workgroup copies its share, so
    // that the copies are done by the last round (the one-shot form's own chunk) and overlap the
    // other workgroups' tiles.
    const unsigned long long all = a.cp.bytes * (unsigned long long)a.cp.n;
    unsigned piece = 64u << 10;
    while (piece < (1u << 20) && (unsigned long long)piece * (unsigned long long)grid < all)
      piece *= 2;
    a.cp.piece_bytes = piece;
    a.cp.pieces = (unsigned)((a.cp.bytes + a.cp.piece_bytes - 1) / a.cp.piece_bytes);
    const long long rounds = std::max(1, (total + grid - 1) / grid - 1);
    const long long pieces = (long long)a.cp.pieces * a.cp.n;
    a.copy_quota = (int)((pieces + grid * rounds - 1) / (grid * rounds));
  }
  if (debug_enabled())
    fprintf(stderr, "[ringag] %s tp=%d s=%d T=%d Kl=%d Mo=%d tile=%dx%d tiles=%d grid=%d "
            "arrive=%d\n", fn, tp, self_rank, T, Kl, Mo, bi, bj, total, grid, (int)arrive);
  if (a.copies) {
    const int rc = join_side_copies(c, stream);
    if (rc) return rc;
  }
  hipEvent_t ev0, ev1;
  launch_timing_events(c, &ev0, &ev1);
  HIPCHK(launch_gemm_rs(c->device, a, tile, grid, stream, ev0, ev1));
  launch_timed(c, ev0);
  if (join) HIPCHK(hipStreamWaitEvent(stream, c->ev_join, 0));
  return RAG_OK;
}

}  // namespace

extern "C" {

int rag_version(void) { return 100; }

const char* rag_last_error(void) { return g_last_error; }

int rag_create(rag_ctx** out, int device, int max_tp, int flags) {
  if (!out) return fail(RAG_EINVAL, "rag_create: out is NULL");
  *out = nullptr;
  if (max_tp < 1 || max_tp > RAG_MAX_TP)
    return fail(RAG_EINVAL, "rag_create: max_tp=%d outside [1, %d]", max_tp, RAG_MAX_TP);
  if (flags != 0) return fail(RAG_EINVAL, "rag_create: flags must be 0 (got %d)", flags);
  int ndev = 0;
  HIPCHK(hipGetDeviceCount(&ndev));
  if (device < 0 || device >= ndev)
    return fail(RAG_EINVAL, "rag_create: device %d outside [0, %d)", device, ndev);
  HIPCHK(hipSetDevice(device));
  hipDeviceProp_t prop;
  HIPCHK(hipGetDeviceProperties(&prop, device));
  if (strncmp(prop.gcnArchName, "gfx950", 6) != 0)
    return fail(RAG_EINVAL, "rag_create: device %d is %s; this library is built for gfx950",
                device, prop.gcnArchName);
  rag_ctx* c = new rag_ctx();
  c->device = device;
  c->max_tp = max_tp;
  c->num_cus = prop.multiProcessorCount;
  int khz = 0;
  if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, device) == hipSuccess && khz > 0)
    c->wall_khz = khz;
  const size_t nwords = ((size_t)max_tp + 1 + 4 * (size_t)kArrSlots + 1) * kWordStride;
  hipError_t e = load_kernels(device);
  if (e != hipSuccess) {
    delete c;
    return fail(RAG_EHIP, "rag_create: loading the gfx950 kernels on device %d failed: %s", device,
                hipGetErrorString(e));
  }
  e = hipStreamCreateWithFlags(&c->side, hipStreamNonBlocking);
  if (e == hipSuccess) e = hipEventCreateWithFlags(&c->ev_fork, hipEventDisableTiming);
  if (e == hipSuccess) e = hipEventCreateWithFlags(&c->ev_join, hipEventDisableTiming);
  if (e == hipSuccess) e = hipEventCreateWithFlags(&c->ev_ag, hipEventDisableTiming);
  if (e == hipSuccess) e = hipEventCreateWithFlags(&c->ev_side, hipEventDisableTiming);
  if (e == hipSuccess) e = hipMalloc((void**)&c->words, nwords * sizeof(int));
  if (e == hipSuccess) e = hipMemset(c->words, 0, nwords * sizeof(int));
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e != hipSuccess) {
    std::string msg = std::string("rag_create: ") + hipGetErrorString(e);
    rag_destroy(c);
    return fail(RAG_EHIP, "%s", msg.c_str());
  }
  c->w.ctr = c->words;
  c->w.arr = reinterpret_cast<unsigned*>(c->words + (size_t)(max_tp + 1) * kWordStride);
  c->w.err = c->words + (size_t)(max_tp + 1 + 4 * kArrSlots) * kWordStride;
  {
    const int rc = setup_scratch_words(device);
    if (rc) {
      rag_destroy(c);
      return rc;
    }
  }
  *out = c;
  if (debug_enabled())
    fprintf(stderr, "[ringag] context on device %d (%s, %d CUs, wall clock %lld kHz), max_tp %d\n",
            device, prop.gcnArchName, c->num_cus, c->wall_khz, max_tp);
  return RAG_OK;
}

int rag_destroy(rag_ctx* c) {
  if (!c) return RAG_OK;
  (void)hipSetDevice(c->device);
  if (c->side) (void)hipStreamSynchronize(c->side);
  for (int q = 0; q < 2; ++q) {
    if (c->sdma[q]) (void)hipStreamSynchronize(c->sdma[q]);
    if (c->sdma[q]) (void)hipStreamDestroy(c->sdma[q]);
    if (c->ev_sdma[q]) (void)hipEventDestroy(c->ev_sdma[q]);
  }
  for (auto ev : c->t_start) (void)hipEventDestroy(ev);
  for (auto ev : c->t_stop) (void)hipEventDestroy(ev);
  for (auto ev : c->ev_chunk) (void)hipEventDestroy(ev);
  if (c->ev_fork) (void)hipEventDestroy(c->ev_fork);
  if (c->ev_join) (void)hipEventDestroy(c->ev_join);
  if (c->ev_ag) (void)hipEventDestroy(c->ev_ag);
  if (c->ev_side) (void)hipEventDestroy(c->ev_side);
  if (c->side) (void)hipStreamDestroy(c->side);
  if (c->words) (void)hipFree(c->words);
  if (c->gbuf) (void)hipFree(c->gbuf);
  if (c->stage) (void)hipFree(c->stage);
  if (c->rsbuf) (void)hipFree(c->rsbuf);
  if (c->slab_flags) (void)hipFree(c->slab_flags);
  delete c;
  return RAG_OK;
}

int rag_set_option(rag_ctx* c, int key, long long v) {
  if (!c) return fail(RAG_EINVAL, "rag_set_option: ctx is NULL");
  switch (key) {
    case RAG_OPT_COPY_ENGINE:
      if (v != RAG_COPY_KERNEL && v != RAG_COPY_SDMA && v != RAG_COPY_IN_GEMM &&
          v != RAG_COPY_IN_GEMM_ASSIST && v != RAG_COPY_IN_GEMM_SDMA)
        return fail(RAG_EINVAL, "copy engine must be 0 (kernel), 1 (sdma), 2 (in the GEMM), 3 "
                    "(in the GEMM with a copy kernel assisting) or 4 (in the GEMM with SDMA for "
                    "the late chunks), got %lld", v);
      c->copy_engine = (int)v;
      return RAG_OK;
    case RAG_OPT_COMM_CUS: {
      if (v != 0 && (v < 8 || v > c->num_cus - 8 || v % 8))
        return fail(RAG_EINVAL, "comm CUs must be 0 (off) or a multiple of 8 in [8, %d], got %lld",
                    c->num_cus - 8, v);
      if (v == c->comm_cus) return RAG_OK;
      // replace the side stream: after its work is done, by one limited to the lowest v
      // compute-unit mask bits (bit b is compute unit b / 8 of XCD b % 8 on gfx950, so every XCD
      // gets v / 8), or by an unrestricted one
      HIPCHK(hipSetDevice(c->device));
      HIPCHK(hipStreamSynchronize(c->side));
      hipStream_t ns = nullptr;
      if (v == 0) {
        HIPCHK(hipStreamCreateWithFlags(&ns, hipStreamNonBlocking));
      } else {
        std::vector<uint32_t> mask((size_t)(c->num_cus + 31) / 32, 0u);
        for (long long b = 0; b < v; ++b) mask[(size_t)b / 32] |= 1u << (b % 32);
        HIPCHK(hipExtStreamCreateWithCUMask(&ns, (uint32_t)mask.size(), mask.data()));
      }
      HIPCHK(hipStreamDestroy(c->side));
      c->side = ns;
      c->side_pending = false;
      c->comm_cus = (int)v;
      return RAG_OK;
    }
    case RAG_OPT_SDMA_STREAMS:
      if (v < 1 || v > 3) return fail(RAG_EINVAL, "SDMA streams must be in [1, 3], got %lld", v);
      HIPCHK(hipSetDevice(c->device));
      for (int q = 0; q + 1 < v; ++q) {
        if (!c->sdma[q]) HIPCHK(hipStreamCreateWithFlags(&c->sdma[q], hipStreamNonBlocking));
        if (!c->ev_sdma[q]) HIPCHK(hipEventCreateWithFlags(&c->ev_sdma[q], hipEventDisableTiming));
      }
      c->sdma_streams = (int)v;
      return RAG_OK;
    case RAG_OPT_COMM_WGS:
      if (v < 1 || v > 1024) return fail(RAG_EINVAL, "comm workgroups must be in [1, 1024]");
      c->comm_wgs = (int)v;
      return RAG_OK;
    case RAG_OPT_SPIN_LIMIT_US:
      if (v < 1 || v > 60000000LL) return fail(RAG_EINVAL, "spin limit must be in [1, 6e7] us");
      c->spin_us = v;
      return RAG_OK;
    case RAG_OPT_ARRIVAL_DELAY_US:
      if (v < 0 || v > 1000000LL) return fail(RAG_EINVAL, "arrival delay must be in [0, 1e6] us");
      c->delay_us = v;
      return RAG_OK;
    case RAG_OPT_WITHHOLD_MASK:
      if (v < 0 || v > 0xffffLL) return fail(RAG_EINVAL, "withhold mask must fit in 16 bits");
      c->withhold = (unsigned)v;
      return RAG_OK;
    case RAG_OPT_TIMING:
      if (v != 0 && v != 1) return fail(RAG_EINVAL, "timing must be 0 or 1");
      if (v && c->t_start.empty()) {
        HIPCHK(hipSetDevice(c->device));
        c->t_start.resize(kTimingSlots);
        c->t_stop.resize(kTimingSlots);
        for (int i = 0; i < kTimingSlots; ++i) {
          HIPCHK(hipEventCreate(&c->t_start[i]));
          HIPCHK(hipEventCreate(&c->t_stop[i]));
        }
      }
      c->timing = v != 0;
      return RAG_OK;
    case RAG_OPT_WGS_PER_CU:
      if (v < 0 || v > 16) return fail(RAG_EINVAL, "workgroups per CU must be in [0, 16]");
      c->wgs_per_cu = (int)v;
      return RAG_OK;
    case RAG_OPT_GEMM_COPY_WGS:
      if (v < 0 || v > 65536) return fail(RAG_EINVAL, "GEMM copy workgroups must be in [0, 65536]");
      c->gemm_copy_wgs = (int)v;
      return RAG_OK;
    case RAG_OPT_AG_GATE:
      if (v != RAG_GATE_CHUNK && v != RAG_GATE_SLAB)
        return fail(RAG_EINVAL, "AG gate must be 0 (whole chunks) or 1 (K slabs), got %lld", v);
      c->ag_gate = (int)v;
      return RAG_OK;
    case RAG_OPT_SLAB_HELP_US:
      if (v < 0 || v > 10000000LL) return fail(RAG_EINVAL, "slab help time must be in [0, 1e7] us");
      c->slab_help_us = v;
      return RAG_OK;
    case RAG_OPT_COPY_PRIORITY:
      if (v != 0 && v != 1) return fail(RAG_EINVAL, "copy priority must be 0 or 1");
      c->copy_priority = (int)v;
      return RAG_OK;
    case RAG_OPT_TRACE_BUF:
      if (v != 0 && (v & 7)) return fail(RAG_EINVAL, "trace buffer must be 8-byte aligned");
      if (v != 0 && !on_device(reinterpret_cast<const void*>(v), c->device))
        return fail(RAG_EINVAL, "trace buffer is not device memory of device %d", c->device);
      c->trace_buf = (unsigned long long)v;
      return RAG_OK;
    case RAG_OPT_TRACE_BYTES:
      if (v < 0) return fail(RAG_EINVAL, "trace size must be >= 0");
      c->trace_bytes = v;
      return RAG_OK;
    case RAG_OPT_TILE:
      if (v < RAG_TILE_AUTO || v > RAG_TILE_256x192_8W) return fail(RAG_EINVAL, "unknown tile %lld", v);
      c->tile = (int)v;
      return RAG_OK;
    default:
      return fail(RAG_EINVAL, "rag_set_option: unknown key %d", key);
  }
}

int ag_gemm(rag_ctx* c, const void* A, int M, int K, const void* const* B, int nc, int tp,
            int self_rank, void* G, void* D, rag_dtype dt, const float* scale_A,
            const float* scale_B, int flags, void* stream_v) {
  return ag_gemm_ex(c, A, M, K, B, nc, tp, self_rank, G, D, dt, scale_A, scale_B, RAG_BF16,
                    nullptr, nullptr, nullptr, flags, stream_v);
}

}  // extern "C"

namespace {

// ag_gemm_ex on the device words W (the context's own, or a device's fixed scratch).
int ag_call(rag_ctx* c, Words& W, const char* fn, const void* A, int M, int K,
            const void* const* B, int nc, int tp, int self_rank, void* G, void* D, rag_dtype dt, const float* scale_A,
            const float* scale_B, rag_dtype d_dt, const float* scale_D, float* amax_D,
            void* B_copy, int flags, void* stream_v) {
  if (tp < 1 || tp > c->max_tp)
    return fail(RAG_EINVAL, "%s: tp=%d outside [1, %d] (max_tp of the context)", fn, tp,
                c->max_tp);
  if (self_rank < 0 || self_rank >= tp)
    return fail(RAG_EINVAL, "%s: self_rank=%d outside [0, tp=%d)", fn, self_rank, tp);
  if (dt != RAG_BF16 && dt != RAG_FP8_E4M3)
    return fail(RAG_EINVAL, "%s: unknown dtype %d", fn, dt);
  const bool fp8 = dt == RAG_FP8_E4M3;
  const int esz = fp8 ? 1 : 2;
  const int kmul = fp8 ? 128 : 64;
  if (M < 1 || nc < 1 || K < 1)
    return fail(RAG_EINVAL, "%s: M=%d, K=%d, nc=%d must all be >= 1", fn, M, K, nc);
  if (K % kmul)
    return fail(RAG_EINVAL, "%s: K=%d must be a multiple of %d for %s", fn, K, kmul,
                fp8 ? "fp8" : "bf16");
  if (flags & ~(RAG_STAGED_OUT | RAG_NO_COPY | RAG_COPY_ONLY | RAG_PER_CHUNK))
    return fail(RAG_EINVAL, "%s: unknown flag bits 0x%x", fn, flags);
  if ((flags & RAG_NO_COPY) && (flags & RAG_COPY_ONLY))
    return fail(RAG_EINVAL, "%s: RAG_NO_COPY and RAG_COPY_ONLY exclude each other", fn);
  if (!A || !B || !D) return fail(RAG_EINVAL, "%s: A, B_chunks and D must not be NULL", fn);
  for (int r = 0; r < tp; ++r) {
    if (!B[r]) return fail(RAG_EINVAL, "%s: B_chunks[%d] is NULL", fn, r);
    if (misaligned(B[r])) return fail(RAG_EINVAL, "%s: B_chunks[%d] is not 16-byte aligned", fn, r);
  }
  if (misaligned(A) || misaligned(D) || (G && misaligned(G)))
    return fail(RAG_EINVAL, "%s: A, G and D must be 16-byte aligned", fn);
  if (fp8 && (!scale_A || !scale_B))
    return fail(RAG_EINVAL, "%s: fp8 needs scale_A and scale_B", fn);
  if (!fp8 && (scale_A || scale_B))
    return fail(RAG_EINVAL, "%s: scales are only meaningful for fp8; pass NULL for bf16", fn);
  if (d_dt != RAG_BF16 && d_dt != RAG_FP8_E4M3)
    return fail(RAG_EINVAL, "%s: unknown output dtype %d", fn, d_dt);
  const bool out8 = d_dt == RAG_FP8_E4M3;
  const int oesz = out8 ? 1 : 2;
  if (out8 && !scale_D) return fail(RAG_EINVAL, "%s: fp8 output needs scale_D", fn);
  if (!out8 && (scale_D || amax_D))
    return fail(RAG_EINVAL, "%s: scale_D and amax_D are only meaningful for fp8 output", fn);
  if ((amax_D && (reinterpret_cast<uintptr_t>(amax_D) & 3u)) || (B_copy && misaligned(B_copy)))
    return fail(RAG_EINVAL, "%s: amax_D must be 4-byte and B_copy 16-byte aligned", fn);
  {
    HIPCHK(hipSetDevice(c->device));
    const void* named[] = {A, D, G, scale_A, scale_B, scale_D, amax_D, B_copy};
    const char* names[] = {"A", "D", "G", "scale_A", "scale_B", "scale_D", "amax_D", "B_copy"};
    for (int i = 0; i < 8; ++i)
      if (named[i] && !on_device(named[i], c->device))
        return fail(RAG_EINVAL, "%s: %s is not device memory of device %d", fn, names[i],
                    c->device);
    for (int r = 0; r < tp; ++r)
      if (!on_device(B[r], c->device))
        return fail(RAG_EINVAL, "%s: B_chunks[%d] is not device memory of device %d", fn, r,
                    c->device);
  }
  const long long a_bytes = (long long)M * K * esz;
  const long long chunk_bytes = (long long)nc * K * esz;
  const long long g_bytes = chunk_bytes * tp;
  const long long d_bytes = (long long)tp * nc * M * oesz;
  if (a_bytes > kMaxOperandBytes || chunk_bytes > kMaxOperandBytes)
    return fail(RAG_EINVAL, "%s: the weight (%lld B) and each chunk (%lld B) must be < 2 GiB", fn,
                a_bytes, chunk_bytes);
  if (overlaps(D, d_bytes, A, a_bytes) || (G && overlaps(G, g_bytes, A, a_bytes)) ||
      (G && overlaps(G, g_bytes, D, d_bytes)))
    return fail(RAG_EINVAL, "%s: G and D must not overlap A or each other", fn);
  for (int r = 0; r < tp; ++r)
    if (overlaps(D, d_bytes, B[r], chunk_bytes) ||
        (G && r != self_rank && overlaps(G, g_bytes, B[r], chunk_bytes)))
      return fail(RAG_EINVAL, "%s: G and D must not overlap B_chunks[%d]", fn, r);
  if (B_copy) {
    if (overlaps(B_copy, chunk_bytes, A, a_bytes) || overlaps(B_copy, chunk_bytes, D, d_bytes) ||
        (G && overlaps(B_copy, chunk_bytes, G, g_bytes)))
      return fail(RAG_EINVAL, "%s: B_copy must not overlap A, G or D", fn);
    for (int r = 0; r < tp; ++r)
      if (overlaps(B_copy, chunk_bytes, B[r], chunk_bytes))
        return fail(RAG_EINVAL, "%s: B_copy must not overlap B_chunks[%d]", fn, r);
  }
  if (G && overlaps(G, g_bytes, B[self_rank], chunk_bytes) &&
      (const char*)B[self_rank] != (const char*)G + (size_t)self_rank * chunk_bytes)
    return fail(RAG_EINVAL, "%s: the own chunk may only sit in G at its own slot", fn);
  if ((flags & RAG_NO_COPY) && !G && !c->gbuf)
    return fail(RAG_EINVAL, "%s: RAG_NO_COPY reads the chunks from G; pass G", fn);
  if ((c->copy_engine == RAG_COPY_SDMA || c->copy_engine == RAG_COPY_IN_GEMM_SDMA) &&
      c->delay_us > 0 && !(flags & RAG_NO_COPY))
    return fail(RAG_EINVAL, "%s: the arrival delay hook needs a compute-unit copy engine", fn);

  HIPCHK(hipSetDevice(c->device));
  hipStream_t stream = (hipStream_t)stream_v;
  const bool staged = (flags & RAG_STAGED_OUT) != 0;
  const bool no_copy = (flags & RAG_NO_COPY) != 0;
  const bool copy_only = (flags & RAG_COPY_ONLY) != 0;

  char* Gp = (char*)G;
  if (!Gp) {
    int rc = ensure_buffer(&c->gbuf, &c->gbuf_bytes, (size_t)g_bytes, "gather buffer");
    if (rc) return rc;
    Gp = (char*)c->gbuf;
  }
  // the own chunk also goes into G (after the peers' chunks) unless it is already there
  const bool own_copy = G && (const char*)B[self_rank] != Gp + (size_t)self_rank * chunk_bytes;
  if (staged && !copy_only) {
    int rc = ensure_buffer(&c->stage, &c->stage_bytes, (size_t)(tp + 1) * nc * M * oesz,
                           "staging buffer");
    if (rc) return rc;
  }
  // Who runs the copies of the simulated arrival: the GEMM launch's own workgroups (in-GEMM,
  // in-GEMM with assist), a copy kernel on the side stream beside the GEMM (kernel, in-GEMM with
  // assist: both take pieces from the same queue), or SDMA on up to three side streams.
  const int engine = c->copy_engine;
  AgPlan plan;
  {
    const int rc = plan_ag(c, nc, M, tp, fp8, out8, no_copy, &plan);
    if (rc) return rc;
  }
  plan_slab(c, nc, K, tp, fp8, copy_only, &W == &c->w, Gp, &plan);
  if (plan.slab.on) {
    // the pieces' flags, zeroed when (re)allocated: they hold past epochs only
    const size_t need = sizeof(int) * (size_t)(tp - 1) * plan.slab.groups * plan.slab.ppc;
    if (c->slab_flags_bytes < need) {
      int rc = ensure_buffer((void**)&c->slab_flags, &c->slab_flags_bytes, need,
                             "slab flags");
      if (rc) return rc;
      HIPCHK(hipMemset(c->slab_flags, 0, need));
    }
    plan.slab.flags = c->slab_flags;
  }
  const bool assist = plan.assist, gemm_copies = plan.gemm_copies, sdma = plan.sdma;
  const bool side_kernel = plan.side_kernel;
  // SDMA beside in-GEMM copies takes only the late peers; the GEMM's workgroups copy the rest
  // (the early peers, the own chunk, B_copy)
  const bool hybrid = plan.hybrid && sdma;
  const int tile = plan.tile, tiles_i = plan.tiles_i, tiles_j = plan.tiles_j, grid = plan.grid;
  const int late = plan.late;
  const bool side = side_kernel || sdma;
  const int epoch = next_epoch(W);
  unsigned long long* trace = nullptr;
  if (c->trace_buf) {
    int bi, bj;
    tile_dims(tile, &bi, &bj);
    const long long tiles = (long long)((nc + bi - 1) / bi) * ((M + bj - 1) / bj) * tp;
    if ((kTraceHeader + kTraceTileWords * tiles) * 8 <= c->trace_bytes)
      trace = reinterpret_cast<unsigned long long*>(c->trace_buf);
  }
  int order[kMaxTp];
  for (int j = 0; j < tp; ++j) order[j] = ((self_rank - j) % tp + tp) % tp;

  if (flags & RAG_PER_CHUNK) {
    const int rc = ag_gemm_split(c, W, A, M, K, B, nc, tp, self_rank, Gp, own_copy, D, fp8,
                                 scale_A, scale_B, out8, scale_D, amax_D, B_copy, staged, no_copy,
                                 copy_only, chunk_bytes, order, epoch, stream);
    if (rc) return rc;
    return staged && !copy_only ? finalize_staged(c, D, nc, M, tp, order, oesz, stream) : RAG_OK;
  }

  // The copies: the peers' chunks in ring order (the last `late` of them the assisting kernel's
  // queue), then the own chunk into G, then B_copy.
  CopyPlan cp = {};
  if (!no_copy) {
    int n = 0;
    for (int j = 1; j < tp; ++j, ++n) {
      const int r = order[j];
      cp.src[n] = B[r];
      cp.dst[n] = Gp + (size_t)r * chunk_bytes;
      cp.ctr_index[n] = r;
      cp.pos[n] = j;
    }
    cp.n_peer = n;
    if (own_copy) {
      cp.src[n] = B[self_rank];
      cp.dst[n] = Gp + (size_t)self_rank * chunk_bytes;
      // when something on a side stream may copy it, the GEMM waits for it before exiting (with
      // B_copy too, or with no GEMM, the caller's stream waits for the side streams instead);
      // when only the GEMM's own workgroups copy it, they finish it before the launch ends
      cp.ctr_index[n] = (copy_only || !side || hybrid || B_copy) ? -1 : c->max_tp;
      cp.pos[n] = 0;
      ++n;
    }
    if (B_copy) {   // this rank's chunk saved for the backward pass
      cp.src[n] = B[self_rank];
      cp.dst[n] = B_copy;
      cp.ctr_index[n] = -1;
      cp.pos[n] = 0;
      ++n;
    }
    cp.n = n;
    cp.late = late;
    cp.late_external = hybrid ? 1 : 0;
    cp.bytes = (unsigned long long)chunk_bytes;
    // a piece is two rounds of 8 16-byte vectors per thread of the GEMM's copying workgroups
    // (or of the copy kernel's, when only it copies)
    cp.piece_bytes = (unsigned)(gemm_copies ? tile_threads(tile) : kArrivalThreads) * 256u;
    cp.pieces = (unsigned)((cp.bytes + cp.piece_bytes - 1) / cp.piece_bytes);
    use_count_set(W, cp);
    cp.delay_ticks = c->delay_us * c->wall_khz / 1000;
    cp.withhold_mask = c->withhold;
    cp.trace = trace;
  }
  // A launch that copies on the caller's stream clears the piece counts a previous call's copy
  // kernel may still use: join it first (before this call's own side-stream kernel is forked)
  if (gemm_copies && cp.n > 0) {
    const int rc = join_side_copies(c, stream);
    if (rc) return rc;
  }
  bool copied = false;   // a launch used this call's set of piece counts
  // the copies SDMA makes: all of them, or with in-GEMM copies beside only the late peers
  const int sdma_first = hybrid ? cp.n_peer - late : 0;
  const int sdma_end = hybrid ? cp.n_peer : cp.n;
  const int nsdma = sdma ? std::min(c->sdma_streams, std::max(1, sdma_end - sdma_first)) : 0;
  if (side) {
    HIPCHK(hipEventRecord(c->ev_fork, stream));
    HIPCHK(hipStreamWaitEvent(c->side, c->ev_fork, 0));
    if (side_kernel) {
      ArrivalArgs aa = {};
      aa.cp = cp;
      aa.ctr = W.ctr;
      aa.epoch = epoch;
      aa.raise_priority = c->copy_priority;
      aa.late_only = assist ? 1 : 0;
      if (cp.n > 0) {
        HIPCHK(launch_arrival(c->device, aa, c->comm_wgs, c->side));
        copied = true;
        const int rc = note_side_copies(c);
        if (rc) return rc;
      }
    } else {
      // SDMA: copy k on side stream k mod nsdma, each followed by its counter's release
      for (int q = 1; q < nsdma; ++q) HIPCHK(hipStreamWaitEvent(c->sdma[q - 1], c->ev_fork, 0));
      for (int k = sdma_first; k < sdma_end; ++k) {
        const int q = (k - sdma_first) % nsdma;
        hipStream_t sk = q == 0 ? c->side : c->sdma[q - 1];
        HIPCHK(hipMemcpyAsync(cp.dst[k], cp.src[k], (size_t)chunk_bytes,
                              hipMemcpyDeviceToDeviceNoCU, sk));
        if (cp.ctr_index[k] >= 0 && (cp.pos[k] == 0 || !((c->withhold >> cp.pos[k]) & 1u)))
          HIPCHK(hipStreamWriteValue32(sk, W.ctr + (size_t)cp.ctr_index[k] * kWordStride,
                                       (uint32_t)epoch, 0));
      }
    }
    // With a GEMM the join is on the device (its workgroups wait for the last copy before they
    // exit); without one, or with B_copy (two copies after the peers', completing in any order),
    // the caller's stream waits for the side streams' ends.
    if (copy_only || B_copy) {
      HIPCHK(hipEventRecord(c->ev_join, c->side));
      for (int q = 1; q < nsdma; ++q) HIPCHK(hipEventRecord(c->ev_sdma[q - 1], c->sdma[q - 1]));
    }
  }

  if (!copy_only || gemm_copies) {
    AgArgs a = {};
    for (int j = 0; j < tp; ++j) {
      const int r = order[j];
      a.chunk[j] = (j == 0) ? B[self_rank] : (const void*)(Gp + (size_t)r * chunk_bytes);
      a.ctr_index[j] = (j == 0 || no_copy) ? -1 : r;
      a.out[j] = (staged && !copy_only) ? (void*)((char*)c->stage + (size_t)j * nc * M * oesz)
                                        : (void*)((char*)D + (size_t)r * nc * M * oesz);
    }
    a.A = A;
    a.M = M;
    a.K = K;
    a.nc = nc;
    a.tp = tp;
    a.ctr = W.ctr;
    a.join_index = (own_copy && side && !hybrid && !B_copy && !copy_only) ? c->max_tp : -1;
    a.epoch = epoch;
    a.err = W.err;
    a.spin_limit = c->spin_us * c->wall_khz / 1000;
    a.scale_A = scale_A;
    a.scale_B = scale_B;
    a.trace = trace ? trace + kTraceHeader : nullptr;
    a.copies = gemm_copies && cp.n > 0;
    a.compute = copy_only ? 0 : 1;
    a.out_fp8 = out8 ? 1 : 0;
    a.scale_D = scale_D;
    a.amax_D = amax_D;
    a.cp = cp;
    a.slab = plan.slab;
    a.tiles_i = tiles_i;
    a.tiles_j = tiles_j;
    const int total = tiles_i * tiles_j * tp;
    // in-kernel copies: workgroups w with (w / 8) % copy_stride == 0 take part (workgroup 0 always)
    a.copy_stride = 1;
    if (a.copies && c->gemm_copy_wgs > 0 && grid >= 8)
      a.copy_stride = std::max(1, (grid / 8) / std::max(1, c->gemm_copy_wgs / 8));
    if (debug_enabled())
      fprintf(stderr, "[ringag] ag_gemm tp=%d s=%d nc=%d K=%d M=%d %s %s tiles=%d grid=%d "
              "(blocks/CU %d, VGPRs %d, LDS %d) engine=%s late=%d comm_wgs=%d pieces=%ux%u B "
              "slab=%d (groups %d, pieces %d, q %d, pre %d) flags=0x%x epoch=%d\n",
              tp, self_rank, nc, K, M, fp8 ? "fp8" : "bf16",
              ag_kernel_name(tile, fp8, out8, a.slab.on != 0), total, grid,
              c->ag_info[tile][fp8][out8].max_blocks_per_cu,
              c->ag_info[tile][fp8][out8].vgprs_per_wave, c->ag_info[tile][fp8][out8].lds_bytes,
              engine_name(engine), late, c->comm_wgs, cp.pieces, cp.piece_bytes, a.slab.on,
              a.slab.groups, a.slab.total, a.slab.q, a.slab.pre, flags, epoch);
    hipEvent_t ev0, ev1;
    launch_timing_events(c, &ev0, &ev1);
    HIPCHK(launch_ag_gemm(c->device, a, tile, fp8, grid, stream, ev0, ev1));
    launch_timed(c, ev0);
    copied = copied || a.copies;
  }
  if (copied) W.arr_seq++;
  if (side && (copy_only || B_copy)) {
    HIPCHK(hipStreamWaitEvent(stream, c->ev_join, 0));
    for (int q = 1; q < nsdma; ++q) HIPCHK(hipStreamWaitEvent(stream, c->ev_sdma[q - 1], 0));
    if (side_kernel) c->side_pending = false;
  }

  return staged && !copy_only ? finalize_staged(c, D, nc, M, tp, order, oesz, stream) : RAG_OK;
}

}  // namespace

extern "C" {

int ag_gemm_ex(rag_ctx* c, const void* A, int M, int K, const void* const* B, int nc, int tp,
               int self_rank, void* G, void* D, rag_dtype dt, const float* scale_A,
               const float* scale_B, rag_dtype d_dt, const float* scale_D, float* amax_D,
               void* B_copy, int flags, void* stream_v) {
  if (!c) return fail(RAG_EINVAL, "ag_gemm: ctx is NULL");
  return ag_call(c, c->w, "ag_gemm", A, M, K, B, nc, tp, self_rank, G, D, dt, scale_A, scale_B,
                 d_dt, scale_D, amax_D, B_copy, flags, stream_v);
}

int ag_gemm_noalloc(rag_ctx* c, const void* A, int M, int K, const void* const* B, int nc,
                    int tp, int self_rank, void* G, void* D, rag_dtype dt, const float* scale_A,
                    const float* scale_B, int flags, void* stream_v) {
  if (!c) return fail(RAG_EINVAL, "ag_gemm_noalloc: ctx is NULL");
  if (tp > kMaxTp)
    return fail(RAG_EINVAL, "ag_gemm_noalloc: tp=%d exceeds the %d ranks the fixed scratch array "
                "holds words for (%d bytes per device)", tp, kMaxTp,
                (int)(sizeof(int) * kScratchWords));
  if (!G)
    return fail(RAG_EINVAL, "ag_gemm_noalloc: G must be given (without it the library would "
                "allocate its own gather buffer)");
  if (flags & (RAG_STAGED_OUT | RAG_PER_CHUNK))
    return fail(RAG_EINVAL, "ag_gemm_noalloc: RAG_STAGED_OUT and RAG_PER_CHUNK are not available "
                "(they use a staging buffer and events the library allocates on first use)");
  Words& W = g_scratch_words[c->device];
  if (!W.ctr)
    return fail(RAG_EINVAL, "ag_gemm_noalloc: the fixed scratch of device %d is not set up",
                c->device);
  return ag_call(c, W, "ag_gemm_noalloc", A, M, K, B, nc, tp, self_rank, G, D, dt, scale_A,
                 scale_B, RAG_BF16, nullptr, nullptr, nullptr, flags, stream_v);
}

int gemm_rs(rag_ctx* c, const void* X, int T, int Kl, const void* W, int Mo,
            const float* const* partials, long long ldp, int tp, int self_rank, float* send,
            void* D, int flags, void* stream_v) {
  return rs_call(c, "gemm_rs", false, X, T, Kl, W, Mo, partials, ldp, tp, self_rank, send, D,
                 flags, stream_v);
}

int gemm_rs_ring(rag_ctx* c, const void* X, int T, int Kl, const void* W, int Mo,
                 const float* const* incoming, long long ldi, int tp, int self_rank, float* send,
                 void* D, int flags, void* stream_v) {
  return rs_call(c, "gemm_rs_ring", true, X, T, Kl, W, Mo, incoming, ldi, tp, self_rank, send, D,
                 flags, stream_v);
}

int linear_allreduce(rag_ctx* c, const void* X, int T, int Kl, const void* W, int Mo,
                     const float* const* partials, long long ldp, const void* const* reduced,
                     int tp, int self_rank, float* send, void* Y, int flags, void* stream_v) {
  if (!c) return fail(RAG_EINVAL, "linear_allreduce: ctx is NULL");
  if (tp < 1 || tp > c->max_tp || self_rank < 0 || self_rank >= tp || T < 1 || T % tp)
    return fail(RAG_EINVAL, "linear_allreduce: tp=%d, self_rank=%d, T=%d do not fit (1 <= tp <= "
                "%d, 0 <= self_rank < tp, T a multiple of tp)", tp, self_rank, T, c->max_tp);
  if (Mo < 8 || Mo % 8) return fail(RAG_EINVAL, "linear_allreduce: Mo=%d must be a multiple of 8", Mo);
  if (!Y || misaligned(Y)) return fail(RAG_EINVAL, "linear_allreduce: Y must be 16-byte aligned");
  const int nc = T / tp;
  const long long cbytes = (long long)nc * Mo * 2;   // one bf16 chunk
  if (tp > 1 && !reduced)
    return fail(RAG_EINVAL, "linear_allreduce: reduced must not be NULL for tp > 1");
  HIPCHK(hipSetDevice(c->device));
  if (!on_device(Y, c->device))
    return fail(RAG_EINVAL, "linear_allreduce: Y is not device memory of device %d", c->device);
  for (int r = 0; r < tp; ++r) {
    if (r == self_rank) continue;
    if (!reduced[r] || misaligned(reduced[r]))
      return fail(RAG_EINVAL, "linear_allreduce: reduced[%d] is NULL or not 16-byte aligned", r);
    if (!on_device(reduced[r], c->device))
      return fail(RAG_EINVAL, "linear_allreduce: reduced[%d] is not device memory of device %d",
                  r, c->device);
    if (overlaps(Y, (long long)T * Mo * 2, reduced[r], cbytes))
      return fail(RAG_EINVAL, "linear_allreduce: Y must not overlap reduced[%d]", r);
  }
  {
    // everything the reduce-scatter checks, before anything is enqueued
    const int rc = rs_call(c, "linear_allreduce", false, X, T, Kl, W, Mo, partials, ldp, tp,
                           self_rank, send, (char*)Y + (size_t)self_rank * cbytes, flags, stream_v,
                           true);
    if (rc) return rc;
    const long long ybytes = (long long)T * Mo * 2;
    if (overlaps(Y, ybytes, X, (long long)T * Kl * 2) || overlaps(Y, ybytes, W, (long long)Mo * Kl * 2) ||
        (send && overlaps(Y, ybytes, send, (long long)T * Mo * 4)))
      return fail(RAG_EINVAL, "linear_allreduce: Y must not overlap X, W or send");
    for (int p = 0; p < tp; ++p)
      if (p != self_rank && overlaps(Y, ybytes, partials[p], ((long long)(T - 1) * ldp + Mo) * 4))
        return fail(RAG_EINVAL, "linear_allreduce: Y must not overlap partials[%d]", p);
  }
  hipStream_t stream = (hipStream_t)stream_v;
  // the all-gather.  With the in-GEMM engine and nothing gated, the GEMM+RS launch copies the
  // owners' reduced chunks itself (after its tiles' epilogues, in ring order); else a copy kernel
  // or SDMA on the side stream, forked before the GEMM so that the copies run beside it.
  if (tp > 1 && in_gemm_engine(c->copy_engine) &&
      !(flags & RAG_RS_ARRIVE)) {
    CopyPlan gp = {};
    int n = 0;
    for (int k = 1; k < tp; ++k, ++n) {
      const int r = ((self_rank - k) % tp + tp) % tp;
      gp.src[n] = reduced[r];
      gp.dst[n] = (char*)Y + (size_t)r * cbytes;
      gp.ctr_index[n] = -1;
      gp.pos[n] = k;
    }
    gp.n_peer = n;
    gp.n = n;
    gp.bytes = (unsigned long long)cbytes;
    gp.piece_bytes = (unsigned)kArrivalThreads * 256u;
    gp.pieces = (unsigned)((gp.bytes + gp.piece_bytes - 1) / gp.piece_bytes);
    return rs_call(c, "linear_allreduce", false, X, T, Kl, W, Mo, partials, ldp, tp, self_rank,
                   send, (char*)Y + (size_t)self_rank * cbytes, flags, stream_v, false, false,
                   &gp);
  }
  if (tp > 1) {
    HIPCHK(hipEventRecord(c->ev_fork, stream));
    HIPCHK(hipStreamWaitEvent(c->side, c->ev_fork, 0));
    if (c->copy_engine == RAG_COPY_SDMA) {
      for (int k = 1; k < tp; ++k) {
        const int r = ((self_rank - k) % tp + tp) % tp;
        HIPCHK(hipMemcpyAsync((char*)Y + (size_t)r * cbytes, reduced[r], (size_t)cbytes,
                              hipMemcpyDeviceToDeviceNoCU, c->side));
      }
    } else {
      ArrivalArgs aa = {};
      int n = 0;
      for (int k = 1; k < tp; ++k, ++n) {
        const int r = ((self_rank - k) % tp + tp) % tp;
        aa.cp.src[n] = reduced[r];
        aa.cp.dst[n] = (char*)Y + (size_t)r * cbytes;
        aa.cp.ctr_index[n] = -1;
        aa.cp.pos[n] = k;
      }
      aa.cp.n_peer = n;
      aa.cp.n = n;
      aa.cp.bytes = (unsigned long long)cbytes;
      aa.cp.piece_bytes = (unsigned)kArrivalThreads * 256u;
      aa.cp.pieces = (unsigned)((aa.cp.bytes + aa.cp.piece_bytes - 1) / aa.cp.piece_bytes);
      use_count_set(c->w, aa.cp);
      aa.ctr = c->w.ctr;
      aa.epoch = c->w.epoch;
      aa.raise_priority = c->copy_priority;
      HIPCHK(launch_arrival(c->device, aa, c->comm_wgs, c->side));
      c->w.arr_seq++;
      const int rc = note_side_copies(c);
      if (rc) return rc;
    }
  }
  // the reduce-scatter of the own chunk, written straight into its slot of Y (with the
  // all-gather's copy kernel running beside it)
  const int rc = rs_call(c, "linear_allreduce", false, X, T, Kl, W, Mo, partials, ldp, tp,
                         self_rank, send, (char*)Y + (size_t)self_rank * cbytes, flags, stream_v,
                         false, tp > 1);
  if (rc) return rc;
  if (tp > 1) {
    // the caller's stream joins everything the side stream ran for this call: the gather's
    // copies, and with RAG_RS_ARRIVE the reduce-scatter's arrivals that rs_call put after them
    HIPCHK(hipEventRecord(c->ev_ag, c->side));
    HIPCHK(hipStreamWaitEvent(stream, c->ev_ag, 0));
    c->side_pending = false;
  }
  return RAG_OK;
}

int rag_ag_kernel_name(rag_ctx* c, int nc, int M, int tp, rag_dtype dt, char* buf, int len) {
  if (!c || !buf || len < 1 || nc < 1 || M < 1 || tp < 1)
    return fail(RAG_EINVAL, "rag_ag_kernel_name: bad arguments");
  if (dt != RAG_BF16 && dt != RAG_FP8_E4M3) return fail(RAG_EINVAL, "unknown dtype %d", dt);
  const bool fp8 = dt == RAG_FP8_E4M3;
  AgPlan plan;
  const int rc = plan_ag(c, nc, M, tp, fp8, false, false, &plan);
  if (rc) return rc;
  // (a call with K = 64, G from the library's own buffer; slab gating does not depend on K
  // otherwise)
  plan_slab(c, nc, 64, tp, fp8, false, true, nullptr, &plan);
  snprintf(buf, (size_t)len, "%s", ag_kernel_name(plan.tile, fp8, false, plan.slab.on != 0));
  return RAG_OK;
}

int rag_rs_kernel_name(rag_ctx* c, int nc, int Mo, int tp, char* buf, int len) {
  if (!c || !buf || len < 1 || nc < 1 || Mo < 1 || tp < 1)
    return fail(RAG_EINVAL, "rag_rs_kernel_name: bad arguments");
  snprintf(buf, (size_t)len, "%s", rs_kernel_name(choose_rs_tile(c, nc, Mo, tp)));
  return RAG_OK;
}

int rag_check(rag_ctx* c) {
  if (!c) return fail(RAG_EINVAL, "rag_check: ctx is NULL");
  HIPCHK(hipSetDevice(c->device));
  HIPCHK(hipDeviceSynchronize());
  // the context's error word, and that of the device's fixed scratch (ag_gemm_noalloc)
  int err = 0, err_s = 0;
  HIPCHK(hipMemcpy(&err, c->w.err, sizeof(int), hipMemcpyDeviceToHost));
  int* serr = g_scratch_words[c->device].err;
  if (serr) HIPCHK(hipMemcpy(&err_s, serr, sizeof(int), hipMemcpyDeviceToHost));
  if (err == 0) err = err_s;
  if (err != 0) {
    HIPCHK(hipMemset(c->w.err, 0, sizeof(int)));
    if (serr) HIPCHK(hipMemset(serr, 0, sizeof(int)));
    HIPCHK(hipDeviceSynchronize());
    return fail(RAG_ETIMEOUT, "a chunk did not arrive within the spin limit (%lld us) in the call "
                "with epoch %d; its tiles were skipped", c->spin_us, err);
  }
  return RAG_OK;
}

int rag_kernel_times(rag_ctx* c, float* out, int max_n) {
  if (!c) return fail(RAG_EINVAL, "rag_kernel_times: ctx is NULL");
  if (max_n < 0 || (max_n > 0 && !out)) return fail(RAG_EINVAL, "rag_kernel_times: bad output");
  HIPCHK(hipSetDevice(c->device));
  const int n = c->n_timed;
  for (int i = 0; i < n; ++i) {
    HIPCHK(hipEventSynchronize(c->t_stop[i]));
    float ms = 0.f;
    HIPCHK(hipEventElapsedTime(&ms, c->t_start[i], c->t_stop[i]));
    if (i < max_n) out[i] = ms;
  }
  c->n_timed = 0;
  return n;
}

}  // extern "C"
