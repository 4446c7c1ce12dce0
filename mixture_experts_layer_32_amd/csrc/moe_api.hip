// libmoe C ABI: validation, buffer layout, launch sequencing and kernel timing.
// Everything a call needs is checked on the host before the first launch; the library never
// allocates device memory and never synchronises the host inside moe_route/moe_fwd/moe_bwd.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <mutex>
#include <string>
#include <vector>

#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

static thread_local std::string g_last_error;

static moe_status fail(moe_status s, const std::string& msg) {
  g_last_error = msg;
  return s;
}

static inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

Layout make_layout(const moe_desc& d) {
  Layout L{};
  L.mx = d.mode == MOE_MODE_MXFP8 || d.mode == MOE_MODE_FP8_BWD || d.mode == MOE_MODE_FP8;
  L.rc = d.recompute != 0;
  L.rows = d.T * (int64_t)d.topk;
  L.nblk_route = (int)((d.T + kRouteTokens - 1) / kRouteTokens);
  L.mtile_cap = (int)(L.rows / kBM) + d.E_local + 1;
  L.mtile2_cap = (int)(L.rows / kBM2) + d.E_local + 1;
  // partial sums of g per pair, one per wave and 256-column tile of the dgrad of h: the fp32 engine's
  // 64-column tiles, the bf16 engine's 4 waves across a tile, the fp8 engine's 2
  L.np = d.mode == MOE_MODE_FP32 ? d.F / 64 : (L.mx ? 2 : 4) * ((d.F + 255) / 256);
  L.elem = d.mode == MOE_MODE_FP32 ? 4 : 2;
  // Pair-contiguous transposed copies (bf16 and fp8 engines): every expert's segment is padded to
  // qpad columns. The bf16 engine reads 64-pair K-tiles; the fp8 engine needs an even number of
  // 64-pair K-tiles per expert and scale rows of a multiple of 4 bytes, hence 128.
  L.qpad = L.mx ? 128 : 64;
  L.qc = d.mode == MOE_MODE_FP32 ? 0 : (L.rows + (int64_t)L.qpad * d.E_local + 127) / 128 * 128;
  const size_t rows = (size_t)L.rows, El = (size_t)d.E_local, T = (size_t)d.T, H = (size_t)d.H, F = (size_t)d.F;
  const size_t qc = (size_t)L.qc;
  // fp8 forward (MXFP8 and blockwise FP8 share every buffer; only the scales' grouping differs)
  const bool mxf = d.mode == MOE_MODE_MXFP8 || d.mode == MOE_MODE_FP8, f8b = d.mode == MOE_MODE_FP8_BWD;
  const bool f32 = d.mode == MOE_MODE_FP32;
  const bool keep = !L.rc;   // the forward leaves its activations in `saved`
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = align256(off + bytes);
    return at;
  };
  L.idx = take(rows * 4);
  L.weight = take(rows * 4);
  L.counts = take(El * 4);
  L.offsets = take((El + 1) * 4);
  L.perm = take(rows * 4);
  L.ptok = take(rows * 4);
  L.pair_pos = take(rows * 4);
  L.mtile = take((size_t)L.mtile_cap * 8);
  L.num_mtiles = take(4);
  L.mtile2 = take((size_t)L.mtile2_cap * 8);
  L.num_mtiles2 = take(4);
  L.zeros = take(kZeroBytes);
  L.qoff = take((El + 1) * 4);
  L.ab = take(keep ? rows * 2 * F * L.elem : 0);
  // w*h row-major: the forward's down GEMM reads it; only the fp32 engine's backward does too, so it
  // stays in `saved` in that mode alone (bf16 modes: forward workspace, hw16 below)
  L.hw = take(keep && f32 ? rows * F * 4 : 0);
  L.hwt = take(keep ? (L.mx ? qc * F : qc * F * 2) : 0);      // MX: E4M3 bytes along the pairs
  L.hwts = take(keep && L.mx ? qc / 32 * F : 0);
  L.sv_wdtq = take(keep && mxf ? El * F * H : 0);
  L.sv_wdts = take(keep && mxf ? El * F * H / 32 : 0);
  L.sv_wgutq = take(keep && mxf ? El * H * 2 * F : 0);
  L.sv_wguts = take(keep && mxf ? El * H * 2 * F / 32 : 0);
  L.saved_total = off;

  off = 0;
  const size_t cells = (size_t)L.nblk_route * El;
  L.sched_f = take(kSchedSlots * kSchedInts * 4);
  L.blk_mask = take(cells * 8);
  L.blk_count = take(cells * 4);
  L.blk_prefix = take(cells * 4);
  L.o = take(rows * H * L.elem);
  L.xq = take(mxf ? T * H : 0);
  L.xs = take(mxf ? T * H / 32 : 0);
  L.wgq = take(mxf ? El * F * H : 0);
  L.wgs = take(mxf ? El * F * H / 32 : 0);
  L.wuq = take(mxf ? El * F * H : 0);
  L.wus = take(mxf ? El * F * H / 32 : 0);
  L.wdq = take(mxf ? El * H * F : 0);
  L.wds = take(mxf ? El * H * F / 32 : 0);
  L.hwq = take(mxf ? rows * F : 0);
  L.hws = take(mxf ? rows * F / 32 : 0);
  L.hw16 = take(d.mode == MOE_MODE_BF16 || f8b ? rows * F * 2 : 0);
  L.f_ab = take(L.rc && f32 ? rows * 2 * F * 4 : 0);    // the fp32 engine writes a, b unconditionally
  L.f_hw = take(L.rc && f32 ? rows * F * 4 : 0);
  L.fwd_total = off;

  off = 0;
  L.sched_b = take(kSchedSlots * kSchedInts * 4);
  L.dab = take(L.mx ? 0 : rows * 2 * F * L.elem);
  L.gpart = take((size_t)L.np * rows * 4);
  L.dxp = take(rows * H * L.elem);
  L.dabt = take(L.mx ? 0 : qc * 2 * F * 2);
  L.dyq = take(L.mx ? T * H : 0);
  L.dys = take(L.mx ? T * H / 32 : 0);
  // the weights quantised along their other axis, when the forward has not left them in `saved`
  const bool wq_here = f8b || (L.rc && mxf);
  L.wdtq = take(wq_here ? El * F * H : 0);
  L.wdts = take(wq_here ? El * F * H / 32 : 0);
  L.wgutq = take(wq_here ? El * H * 2 * F : 0);
  L.wguts = take(wq_here ? El * H * 2 * F / 32 : 0);
  L.dytq = take(L.mx ? H * qc : 0);
  L.dyts = take(L.mx ? H * qc / 32 : 0);
  L.xtq = take(L.mx ? H * qc : 0);
  L.xts = take(L.mx ? H * qc / 32 : 0);
  L.dabq = take(L.mx ? rows * 2 * F : 0);
  L.dabs = take(L.mx ? rows * 2 * F / 32 : 0);
  L.dabtq = take(L.mx ? 2 * F * qc : 0);
  L.dabts = take(L.mx ? 2 * F * qc / 32 : 0);
  L.r_sched = take(L.rc ? kSchedSlots * kSchedInts * 4 : 0);
  L.r_ab = take(L.rc ? rows * 2 * F * L.elem : 0);
  L.r_hw = take(L.rc && f32 ? rows * F * 4 : 0);
  L.r_hwt = take(L.rc ? (L.mx ? qc * F : qc * F * 2) : 0);
  L.r_hwts = take(L.rc && L.mx ? qc / 32 * F : 0);
  L.r_xq = take(L.rc && mxf ? T * H : 0);
  L.r_xs = take(L.rc && mxf ? T * H / 32 : 0);
  L.r_wgq = take(L.rc && mxf ? El * F * H : 0);
  L.r_wgs = take(L.rc && mxf ? El * F * H / 32 : 0);
  L.r_wuq = take(L.rc && mxf ? El * F * H : 0);
  L.r_wus = take(L.rc && mxf ? El * F * H / 32 : 0);
  L.bwd_total = off;
  return L;
}

static moe_status validate(const moe_desc* d) {
  if (!d) return fail(MOE_ERR_INVALID_ARG, "desc is null");
  if (d->T < 1 || d->H < 1 || d->F < 1 || d->E_total < 1 || d->E_local < 1 || d->topk < 1 ||
      d->expert_offset < 0)
    return fail(MOE_ERR_INVALID_ARG, "sizes must be positive (expert_offset >= 0)");
  if (d->topk > d->E_total) return fail(MOE_ERR_INVALID_ARG, "topk exceeds E_total");
  if ((int64_t)d->expert_offset + d->E_local > d->E_total)
    return fail(MOE_ERR_INVALID_ARG, "expert_offset + E_local exceeds E_total");
  if (d->H % 256 != 0) return fail(MOE_ERR_UNSUPPORTED_SHAPE, "H must be a multiple of 256");
  if (d->F % 128 != 0) return fail(MOE_ERR_UNSUPPORTED_SHAPE, "F must be a multiple of 128");
  if (d->E_total > kMaxExperts) return fail(MOE_ERR_UNSUPPORTED_SHAPE, "E_total must be <= 512");
  if (d->topk > kMaxTopk) return fail(MOE_ERR_UNSUPPORTED_SHAPE, "topk must be <= 32");
  if (d->T * (int64_t)d->topk >= (int64_t(1) << 31))
    return fail(MOE_ERR_UNSUPPORTED_SHAPE, "T*topk must be < 2^31");
  if (d->mode != MOE_MODE_FP32 && d->mode != MOE_MODE_BF16 && d->mode != MOE_MODE_MXFP8 &&
      d->mode != MOE_MODE_FP8_BWD && d->mode != MOE_MODE_FP8)
    return fail(MOE_ERR_UNSUPPORTED_MODE, "unknown mode");
  if (d->recompute != 0 && d->recompute != 1) return fail(MOE_ERR_INVALID_ARG, "recompute must be 0 or 1");
  return MOE_OK;
}

static bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

static moe_status check_ptrs(std::initializer_list<std::pair<const void*, const char*>> ps, size_t a) {
  for (auto& q : ps) {
    if (!q.first) return fail(MOE_ERR_INVALID_ARG, std::string(q.second) + " is null");
    if (!aligned(q.first, a))
      return fail(MOE_ERR_INVALID_ARG, std::string(q.second) + " is not " + std::to_string(a) + "-byte aligned");
  }
  return MOE_OK;
}

static moe_status hip_fail(hipError_t e, const char* where) {
  return fail(MOE_ERR_HIP, std::string(where) + ": " + hipGetErrorString(e));
}

static bool kernel_timing_on();

// The work goes to the stream's device, the CU count, the side stream and the static scratch are the
// calling thread's current device's: the two must be the same (the null stream is the current
// device's).
static moe_status check_stream(void* stream) {
  if (!stream) return MOE_OK;
  int cur = 0;
  hipDevice_t sd = 0;
  if (hipGetDevice(&cur) != hipSuccess || hipStreamGetDevice(static_cast<hipStream_t>(stream), &sd) != hipSuccess)
    return fail(MOE_ERR_INVALID_ARG, "stream: its device could not be queried");
  if (sd != cur)
    return fail(MOE_ERR_INVALID_ARG, "stream belongs to device " + std::to_string(sd) +
                                         ", not to the current device " + std::to_string(cur));
  return MOE_OK;
}

// The backward's weight-gradient GEMMs run on a second stream per device, ordered against the
// caller's stream by events, so that their workgroups take the CUs the critical path's kernels free
// at their tails. The stream and its events are created on first use outside a graph capture (no
// side stream then: everything runs in order on the caller's stream). A thread holds the device's
// lock from the fork to the join, so that the events' record/wait pairs of different host threads
// do not interleave, and a side stream taken into one thread's graph capture is back out of it
// before another thread uses it.
namespace {
struct SideStream {
  hipStream_t s = nullptr;
  hipEvent_t fork = nullptr, mid = nullptr, join = nullptr;
  bool tried = false;
  std::mutex mu;
};
SideStream g_side[64];
thread_local SideStream* t_side_pending = nullptr;     // forked and not yet joined by this thread
thread_local std::unique_lock<std::mutex> t_side_lock;  // that device's lock, held until the join
SideStream* side_of_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  return &g_side[dev];
}
}  // namespace

hipStream_t side_stream_fork(hipStream_t s) {
  if (t_side_pending) side_stream_join(s);   // a fork left unjoined: never hold two locks
  // while kernel timing is on, everything stays on s so that each kernel's events bracket it alone
  SideStream* ss = kernel_timing_on() ? nullptr : side_of_device();
  if (!ss) return nullptr;
  std::unique_lock<std::mutex> lk(ss->mu);
  if (!ss->s) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (ss->tried || hipStreamIsCapturing(s, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone) return nullptr;
    ss->tried = true;
    if (hipStreamCreateWithFlags(&ss->s, hipStreamNonBlocking) != hipSuccess ||
        hipEventCreateWithFlags(&ss->fork, hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&ss->mid, hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&ss->join, hipEventDisableTiming) != hipSuccess) {
      ss->s = nullptr;
      return nullptr;
    }
  }
  if (hipEventRecord(ss->fork, s) != hipSuccess || hipStreamWaitEvent(ss->s, ss->fork, 0) != hipSuccess)
    return nullptr;
  t_side_pending = ss;
  t_side_lock = std::move(lk);
  return ss->s;
}

hipError_t side_stream_mark(hipStream_t s) {
  SideStream* ss = t_side_pending;
  return ss ? hipEventRecord(ss->mid, s) : hipSuccess;
}

hipError_t side_stream_wait_mark() {
  SideStream* ss = t_side_pending;
  return ss ? hipStreamWaitEvent(ss->s, ss->mid, 0) : hipSuccess;
}

hipError_t side_stream_join(hipStream_t s) {
  SideStream* ss = t_side_pending;
  if (!ss) return hipSuccess;
  t_side_pending = nullptr;
  std::unique_lock<std::mutex> lk = std::move(t_side_lock);   // released on return
  hipError_t err = hipEventRecord(ss->join, ss->s);
  if (err != hipSuccess) return err;
  return hipStreamWaitEvent(s, ss->join, 0);
}

int persistent_grid(int blocks_per_cu) {
  static int cached_dev = -1, cached_cus = 0;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = 0;
  if (dev != cached_dev) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
    cached_cus = cus;
    cached_dev = dev;
  }
  const int g = (cached_cus * blocks_per_cu) & ~7;
  return g < 8 ? 8 : g;
}

// ------------------------------------------------------------------------------------ profiling
namespace {
struct Prof {
  std::mutex mu;
  bool on = false;
  int cap = 0, n = 0;
  std::vector<hipEvent_t> ev;  // 2 per record
  std::vector<int> rec_kernel;
  std::vector<std::string> names;
  std::vector<int> launches;
  std::vector<double> total_ms;
};
Prof& prof() {
  static Prof p;
  return p;
}
thread_local int t_pending = -1;
}  // namespace

static bool kernel_timing_on() { return prof().on; }

void prof_mark_begin(const char* name, hipStream_t s) {
  Prof& P = prof();
  if (!P.on) return;
  std::lock_guard<std::mutex> g(P.mu);
  if (!P.on || P.n >= P.cap) return;
  int kid = -1;
  for (size_t i = 0; i < P.names.size(); ++i)
    if (P.names[i] == name) kid = (int)i;
  if (kid < 0) {
    P.names.push_back(name);
    P.launches.push_back(0);
    P.total_ms.push_back(0.0);
    kid = (int)P.names.size() - 1;
  }
  if (hipEventRecord(P.ev[2 * P.n], s) == hipSuccess) t_pending = kid;
}

void prof_mark_end(hipStream_t s) {
  Prof& P = prof();
  if (!P.on || t_pending < 0) return;
  std::lock_guard<std::mutex> g(P.mu);
  const int kid = t_pending;
  t_pending = -1;
  if (P.n >= P.cap) return;
  if (hipEventRecord(P.ev[2 * P.n + 1], s) != hipSuccess) return;
  P.rec_kernel[P.n] = kid;
  P.n++;
}

}  // namespace moe

using namespace moe;

extern "C" {

const char* moe_version(void) {
  return "libmoe 0.2 (gfx950; fp32/bf16/mxfp8/fp8_bwd/fp8; persistent grouped GEMM, 256x256 tiles)";
}

const char* moe_status_string(moe_status s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED_SHAPE: return "unsupported shape";
    case MOE_ERR_UNSUPPORTED_MODE: return "unsupported mode";
    case MOE_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case MOE_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* moe_last_error(void) { return g_last_error.c_str(); }

moe_status moe_query_sizes(const moe_desc* d, size_t* fwd_ws, size_t* bwd_ws, size_t* saved) {
  g_last_error.clear();
  moe_status st = validate(d);
  if (st != MOE_OK) return st;
  const Layout L = make_layout(*d);
  if (fwd_ws) *fwd_ws = L.fwd_total;
  if (bwd_ws) *bwd_ws = L.bwd_total;
  if (saved) *saved = L.saved_total;
  return MOE_OK;
}

moe_status moe_saved_layout(const moe_desc* d, moe_saved_offsets* out) {
  g_last_error.clear();
  moe_status st = validate(d);
  if (st != MOE_OK) return st;
  if (!out) return fail(MOE_ERR_INVALID_ARG, "out is null");
  const Layout L = make_layout(*d);
  out->idx = L.idx;
  out->weight = L.weight;
  out->counts = L.counts;
  out->offsets = L.offsets;
  out->perm = L.perm;
  out->pair_pos = L.pair_pos;
  // with activation checkpointing `saved` holds the routing results alone
  const bool act = L.mx && !L.rc;
  const bool mxf = act && (d->mode == MOE_MODE_MXFP8 || d->mode == MOE_MODE_FP8);
  out->qoff = L.mx ? L.qoff : 0;
  out->qcols = L.mx ? (size_t)L.qc : 0;
  out->hwt = act ? L.hwt : 0;
  out->hwt_scales = act ? L.hwts : 0;
  out->wdt = mxf ? L.sv_wdtq : 0;
  out->wdt_scales = mxf ? L.sv_wdts : 0;
  out->wgut = mxf ? L.sv_wgutq : 0;
  out->wgut_scales = mxf ? L.sv_wguts : 0;
  return MOE_OK;
}

static RouteParams route_params(const moe_desc& d, const Layout& L, const float* logits, void* saved, void* ws) {
  char* sv = static_cast<char*>(saved);
  char* w = static_cast<char*>(ws);
  RouteParams p{};
  p.logits = logits;
  p.idx = reinterpret_cast<int*>(sv + L.idx);
  p.weight = reinterpret_cast<float*>(sv + L.weight);
  p.counts = reinterpret_cast<int*>(sv + L.counts);
  p.offsets = reinterpret_cast<int*>(sv + L.offsets);
  p.perm = reinterpret_cast<int*>(sv + L.perm);
  p.ptok = reinterpret_cast<int*>(sv + L.ptok);
  p.pair_pos = reinterpret_cast<int*>(sv + L.pair_pos);
  p.mtile = reinterpret_cast<int2*>(sv + L.mtile);
  p.num_mtiles = reinterpret_cast<int*>(sv + L.num_mtiles);
  p.mtile2 = reinterpret_cast<int2*>(sv + L.mtile2);
  p.num_mtiles2 = reinterpret_cast<int*>(sv + L.num_mtiles2);
  p.zeros = reinterpret_cast<uint4*>(sv + L.zeros);
  p.qoff = reinterpret_cast<int*>(sv + L.qoff);
  p.blk_mask = reinterpret_cast<unsigned long long*>(w + L.blk_mask);
  p.blk_count = reinterpret_cast<int*>(w + L.blk_count);
  p.blk_prefix = reinterpret_cast<int*>(w + L.blk_prefix);
  p.sched = reinterpret_cast<int*>(w + L.sched_f);
  p.T = d.T;
  p.E = d.E_total;
  p.El = d.E_local;
  p.e0 = d.expert_offset;
  p.k = d.topk;
  p.nblk = L.nblk_route;
  p.qpad = L.qpad;
  return p;
}

moe_status moe_route(const moe_desc* d, const float* logits, void* saved, void* ws, size_t ws_bytes,
                     void* stream) {
  g_last_error.clear();
  moe_status st = validate(d);
  if (st != MOE_OK) return st;
  if ((st = check_ptrs({{logits, "logits"}}, 4)) != MOE_OK) return st;
  if ((st = check_ptrs({{saved, "saved"}, {ws, "ws"}}, 256)) != MOE_OK) return st;
  if ((st = check_stream(stream)) != MOE_OK) return st;
  const Layout L = make_layout(*d);
  if (ws_bytes < L.fwd_total) return fail(MOE_ERR_WORKSPACE_TOO_SMALL, "forward workspace too small");
  hipError_t e = launch_route(route_params(*d, L, logits, saved, ws), static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "route launch");
  return MOE_OK;
}

// ------------------------------------------------------------------ routing without a workspace
// moe_route_static: moe_route with its scratch (the per-block token masks, counts and prefixes, and
// the tile-scheduler counters it zeroes) in one file-scope device array instead of a workspace
// argument, for callers that cannot allocate. Every call on a GPU shares that GPU's copy.
constexpr size_t kStaticScratchBytes = size_t(8) << 20;
static __device__ __align__(256) char scratch[kStaticScratchBytes];

// Byte offsets of the routing scratch inside the static array, and the bytes it needs.
struct RouteScratch {
  size_t sched, blk_mask, blk_count, blk_prefix, total;
};
static RouteScratch route_scratch(const moe_desc& d) {
  RouteScratch R{};
  const size_t cells = (size_t)((d.T + kRouteTokens - 1) / kRouteTokens) * (size_t)d.E_local;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = align256(off + bytes);
    return at;
  };
  R.sched = take(kSchedSlots * kSchedInts * 4);
  R.blk_mask = take(cells * 8);
  R.blk_count = take(cells * 4);
  R.blk_prefix = take(cells * 4);
  R.total = off;
  return R;
}

// Device address of `scratch` on the current device, looked up once per device (with that device
// current) and kept: each GPU holds its own copy of the array at its own address. The array's name
// is a host-side stand-in in host code; only this address may reach a kernel.
static moe_status static_scratch(char** out) {
  static std::mutex mu;
  static std::vector<char*> per_device;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  std::lock_guard<std::mutex> g(mu);
  if ((size_t)dev >= per_device.size()) per_device.resize(dev + 1, nullptr);
  if (!per_device[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!ptr) return fail(MOE_ERR_HIP, "hipGetSymbolAddress(scratch) returned a null address");
    per_device[dev] = static_cast<char*>(ptr);
  }
  *out = per_device[dev];
  return MOE_OK;
}

moe_status moe_route_static(const moe_desc* d, const float* logits, void* saved, void* stream) {
  g_last_error.clear();
  moe_status st = validate(d);
  if (st != MOE_OK) return st;
  if ((st = check_ptrs({{logits, "logits"}}, 4)) != MOE_OK) return st;
  if ((st = check_ptrs({{saved, "saved"}}, 256)) != MOE_OK) return st;
  if ((st = check_stream(stream)) != MOE_OK) return st;
  const RouteScratch R = route_scratch(*d);
  if (R.total > kStaticScratchBytes)
    return fail(MOE_ERR_UNSUPPORTED_SHAPE, "moe_route_static needs " + std::to_string(R.total) +
                                               " bytes of scratch (16 per 64 tokens and local expert, plus 512); "
                                               "the static scratch holds " + std::to_string(kStaticScratchBytes));
  char* sc = nullptr;
  if ((st = static_scratch(&sc)) != MOE_OK) return st;
  const Layout L = make_layout(*d);
  // the layout's workspace offsets are replaced by the scratch's; every scratch word the routing
  // reads is written earlier in the same call, so nothing needs clearing
  RouteParams p = route_params(*d, L, logits, saved, sc);
  p.sched = reinterpret_cast<int*>(sc + R.sched);
  p.blk_mask = reinterpret_cast<unsigned long long*>(sc + R.blk_mask);
  p.blk_count = reinterpret_cast<int*>(sc + R.blk_count);
  p.blk_prefix = reinterpret_cast<int*>(sc + R.blk_prefix);
  hipError_t e = launch_route(p, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "route launch");
  return MOE_OK;
}

// The forward after validation: routing (from the given logits, or the router projection fused with
// the top-k when w_router is given, writing the logits to logits_out), then the expert GEMMs and the
// combine.
static moe_status fwd_impl(const moe_desc* d, const void* x, const float* logits, const void* w_router,
                           float* logits_out, const void* w_gate, const void* w_up, const void* w_down, void* y,
                           void* saved, void* ws, size_t ws_bytes, void* stream) {
  moe_status st;
  if ((st = check_ptrs({{x, "x"}, {w_gate, "w_gate"}, {w_up, "w_up"}, {w_down, "w_down"}, {y, "y"}}, 16)) != MOE_OK)
    return st;
  if ((st = check_ptrs({{w_router ? logits_out : logits, "logits"}}, 4)) != MOE_OK) return st;
  if (w_router && (st = check_ptrs({{w_router, "w_router"}}, 16)) != MOE_OK) return st;
  if ((st = check_ptrs({{saved, "saved"}, {ws, "ws"}}, 256)) != MOE_OK) return st;
  if ((st = check_stream(stream)) != MOE_OK) return st;
  const Layout L = make_layout(*d);
  if (ws_bytes < L.fwd_total) return fail(MOE_ERR_WORKSPACE_TOO_SMALL, "forward workspace too small");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const RouteParams rp = route_params(*d, L, w_router ? logits_out : logits, saved, ws);
  hipError_t e = w_router ? launch_router_route_bf16(rp, x, w_router, logits_out, d->H, s) : launch_route(rp, s);
  if (e != hipSuccess) return hip_fail(e, "route launch");
  char* sv = static_cast<char*>(saved);
  FwdParams fp{};
  fp.x = x;
  fp.wg = w_gate;
  fp.wu = w_up;
  fp.wd = w_down;
  fp.perm = rp.perm;
  fp.ptok = rp.ptok;
  fp.offsets = rp.offsets;
  fp.mtile = rp.mtile;
  fp.num_mtiles = rp.num_mtiles;
  fp.mtile2 = rp.mtile2;
  fp.num_mtiles2 = rp.num_mtiles2;
  fp.zeros = rp.zeros;
  fp.sched = rp.sched;
  fp.qoff = rp.qoff;
  fp.qc = L.qc;
  // activation checkpointing: nothing for the backward (it recomputes a, b and hw); only hw, the
  // down GEMM's operand, is written, into the workspace
  fp.hwt = L.rc ? nullptr : sv + L.hwt;
  fp.weight = rp.weight;
  fp.ab = L.rc ? nullptr : sv + L.ab;
  fp.hw = sv + L.hw;
  fp.o = static_cast<char*>(ws) + L.o;
  fp.pair_pos = rp.pair_pos;
  fp.y = y;
  fp.T = d->T;
  fp.H = d->H;
  fp.F = d->F;
  fp.k = d->topk;
  fp.El = d->E_local;
  char* w = static_cast<char*>(ws);
  const int tpw = combine_tpw(d->topk, d->E_local, d->E_total);
  if (d->mode == MOE_MODE_FP32) {
    if (L.rc) {   // the fp32 engine writes a, b and hw unconditionally: workspace scratch
      fp.ab = w + L.f_ab;
      fp.hw = w + L.f_hw;
    }
    if ((e = launch_forward_gemms<float>(fp, persistent_grid(2), s)) != hipSuccess)
      return hip_fail(e, "forward GEMM launch");
    if ((e = launch_combine<float>(fp.o, fp.pair_pos, y, d->T, d->topk, d->H, tpw, s)) != hipSuccess)
      return hip_fail(e, "combine launch");
  } else if (d->mode == MOE_MODE_BF16) {
    fp.hw = w + L.hw16;
    if ((e = launch_forward_gemms_bf16(fp, persistent_grid(1), s)) != hipSuccess)
      return hip_fail(e, "forward GEMM launch");
    if ((e = launch_combine<bf16>(fp.o, fp.pair_pos, y, d->T, d->topk, d->H, tpw, s)) != hipSuccess)
      return hip_fail(e, "combine launch");
  } else if (d->mode == MOE_MODE_MXFP8 || d->mode == MOE_MODE_FP8) {
    // every forward GEMM operand as MXFP8 (blockwise FP8) along its contraction axis; hw and its
    // transposed copy are quantised in the gate/up epilogue. Each weight is read once and quantised
    // along both axes: the other orientation is the backward's operand and goes to `saved`.
    auto u8 = [&](size_t o) { return reinterpret_cast<uint8_t*>(w + o); };
    auto s8 = [&](size_t o) { return reinterpret_cast<uint8_t*>(sv + o); };
    const int El = d->E_local, H = d->H, F = d->F;
    const bool blk = d->mode == MOE_MODE_FP8;
    // with activation checkpointing the backward quantises the weights' other orientation itself
    auto sv8 = [&](size_t o) { return L.rc ? nullptr : s8(o); };
    if ((e = launch_quant_rows(x, u8(L.xq), u8(L.xs), d->T * d->H, "mx_quant_x", s, blk)) != hipSuccess ||
        (e = launch_quant_both(w_gate, u8(L.wgq), u8(L.wgs), sv8(L.sv_wgutq), sv8(L.sv_wguts), El, F, H, 2 * F, 0,
                               "mx_quant_w_gate", s, blk)) != hipSuccess ||
        (e = launch_quant_both(w_up, u8(L.wuq), u8(L.wus), sv8(L.sv_wgutq), sv8(L.sv_wguts), El, F, H, 2 * F, F,
                               "mx_quant_w_up", s, blk)) != hipSuccess ||
        (e = launch_quant_both(w_down, u8(L.wdq), u8(L.wds), sv8(L.sv_wdtq), sv8(L.sv_wdts), El, H, F, H, 0,
                               "mx_quant_w_down", s, blk)) != hipSuccess)
      return hip_fail(e, "quantise launch");
    fp.blk = blk;
    fp.xq = u8(L.xq);
    fp.xs = u8(L.xs);
    fp.wgq = u8(L.wgq);
    fp.wgs = u8(L.wgs);
    fp.wuq = u8(L.wuq);
    fp.wus = u8(L.wus);
    fp.wdq = u8(L.wdq);
    fp.wds = u8(L.wds);
    fp.hwq = u8(L.hwq);
    fp.hws = u8(L.hws);
    fp.hwtq = L.rc ? nullptr : reinterpret_cast<uint8_t*>(sv + L.hwt);
    fp.hwts = L.rc ? nullptr : reinterpret_cast<uint8_t*>(sv + L.hwts);
    if ((e = launch_forward_gemms_mx(fp, persistent_grid(1), s)) != hipSuccess)
      return hip_fail(e, "forward GEMM launch");
    if ((e = launch_combine<bf16>(fp.o, fp.pair_pos, y, d->T, d->topk, d->H, tpw, s)) != hipSuccess)
      return hip_fail(e, "combine launch");
  } else {
    // FP8_BWD: the bf16 forward; its epilogue writes the pair-contiguous hw copy as MXFP8 for the
    // backward's down weight gradient
    fp.hw = w + L.hw16;
    fp.hwtq = L.rc ? nullptr : reinterpret_cast<uint8_t*>(sv + L.hwt);   // null: the bf16 kernel without it
    fp.hwts = L.rc ? nullptr : reinterpret_cast<uint8_t*>(sv + L.hwts);
    if ((e = launch_forward_gemms_bf16(fp, persistent_grid(1), s)) != hipSuccess)
      return hip_fail(e, "forward GEMM launch");
    if ((e = launch_combine<bf16>(fp.o, fp.pair_pos, y, d->T, d->topk, d->H, tpw, s)) != hipSuccess)
      return hip_fail(e, "combine launch");
  }
  return MOE_OK;
}

moe_status moe_fwd(const moe_desc* d, const void* x, const float* logits, const void* w_gate, const void* w_up,
                   const void* w_down, void* y, void* saved, void* ws, size_t ws_bytes, void* stream) {
  g_last_error.clear();
  moe_status st = validate(d);
  if (st != MOE_OK) return st;
  return fwd_impl(d, x, logits, nullptr, nullptr, w_gate, w_up, w_down, y, saved, ws, ws_bytes, stream);
}

moe_status moe_fwd_router(const moe_desc* d, const void* x, const void* w_router, float* logits, const void* w_gate,
                          const void* w_up, const void* w_down, void* y, void* saved, void* ws, size_t ws_bytes,
                          void* stream) {
  g_last_error.clear();
  moe_status st = validate(d);
  if (st != MOE_OK) return st;
  if (d->mode == MOE_MODE_FP32) return fail(MOE_ERR_UNSUPPORTED_MODE, "moe_fwd_router takes bf16 x and w_router");
  if (d->E_total > 256 || d->topk > 8)
    return fail(MOE_ERR_UNSUPPORTED_SHAPE, "moe_fwd_router needs E_total <= 256 and topk <= 8 "
                                           "(else moe_router_fwd, then moe_fwd)");
  return fwd_impl(d, x, nullptr, w_router, logits, w_gate, w_up, w_down, y, saved, ws, ws_bytes, stream);
}

// Activation checkpointing: the gate/up GEMM of the forward again, from x and the weights, with its
// outputs (a and b, and w*h along the pairs: the backward's operands) in the backward workspace. In
// the fp8 modes x and the gate/up weights are quantised again first, and the weights' backward
// orientation is quantised here, since the forward left nothing in `saved`. The same kernels on the
// same inputs give the forward's bits. Points p (the backward's parameters) at the results.
static hipError_t recompute_activations(const moe_desc& d, const Layout& L, BwdParams& p, char* w,
                                        hipStream_t s) {
  auto u8 = [&](size_t o) { return reinterpret_cast<uint8_t*>(w + o); };
  const int El = d.E_local, H = d.H, F = d.F;
  FwdParams fp{};
  fp.x = p.x;
  fp.wg = p.wg;
  fp.wu = p.wu;
  fp.wd = p.wd;
  fp.perm = p.perm;
  fp.ptok = p.ptok;
  fp.offsets = p.offsets;
  fp.mtile = p.mtile;
  fp.num_mtiles = p.num_mtiles;
  fp.mtile2 = p.mtile2;
  fp.num_mtiles2 = p.num_mtiles2;
  fp.zeros = p.zeros;
  fp.qoff = p.qoff;
  fp.qc = L.qc;
  fp.weight = p.weight;
  fp.pair_pos = p.pair_pos;
  fp.sched = reinterpret_cast<int*>(w + L.r_sched);
  fp.ab = w + L.r_ab;
  fp.T = d.T;
  fp.H = H;
  fp.F = F;
  fp.k = d.topk;
  fp.El = El;
  p.ab = fp.ab;
  hipError_t e;
  if (d.mode == MOE_MODE_FP32) {
    fp.hw = w + L.r_hw;
    p.hw = fp.hw;
    return launch_forward_gemms<float>(fp, persistent_grid(2), s, true);
  }
  if (d.mode == MOE_MODE_BF16) {
    fp.hwt = w + L.r_hwt;
    p.hwt = fp.hwt;
    return launch_forward_gemms_bf16(fp, persistent_grid(1), s, true);
  }
  fp.hwtq = u8(L.r_hwt);
  fp.hwts = u8(L.r_hwts);
  if (d.mode == MOE_MODE_FP8_BWD) return launch_forward_gemms_bf16(fp, persistent_grid(1), s, true);
  // MXFP8 / blockwise FP8: x and the gate/up weights along H, and the weights' backward orientation
  const bool blk = d.mode == MOE_MODE_FP8;
  if ((e = launch_quant_rows(p.x, u8(L.r_xq), u8(L.r_xs), d.T * H, "mx_quant_x_recompute", s, blk)) != hipSuccess ||
      (e = launch_quant_both(p.wg, u8(L.r_wgq), u8(L.r_wgs), u8(L.wgutq), u8(L.wguts), El, F, H, 2 * F, 0,
                             "mx_quant_w_gate_recompute", s, blk)) != hipSuccess ||
      (e = launch_quant_both(p.wu, u8(L.r_wuq), u8(L.r_wus), u8(L.wgutq), u8(L.wguts), El, F, H, 2 * F, F,
                             "mx_quant_w_up_recompute", s, blk)) != hipSuccess)
    return e;
  e = blk ? launch_quant_both(p.wd, nullptr, nullptr, u8(L.wdtq), u8(L.wdts), El, H, F, H, 0, "mx_quant_w_down_t", s, true)
          : launch_quant_cols(p.wd, u8(L.wdtq), u8(L.wdts), El, H, F, H, 0, "mx_quant_w_down_t", s);
  if (e != hipSuccess) return e;
  fp.blk = blk;
  fp.xq = u8(L.r_xq);
  fp.xs = u8(L.r_xs);
  fp.wgq = u8(L.r_wgq);
  fp.wgs = u8(L.r_wgs);
  fp.wuq = u8(L.r_wuq);
  fp.wus = u8(L.r_wus);
  return launch_forward_gemms_mx(fp, persistent_grid(1), s, true);
}

moe_status moe_bwd(const moe_desc* d, const void* dy, const void* x, const void* w_gate, const void* w_up,
                   const void* w_down, const void* saved, void* dx, float* dlogits, void* dw_gate, void* dw_up,
                   void* dw_down, void* ws, size_t ws_bytes, void* stream) {
  g_last_error.clear();
  moe_status st = validate(d);
  if (st != MOE_OK) return st;
  if ((st = check_ptrs({{dy, "dy"}, {x, "x"}, {w_gate, "w_gate"}, {w_up, "w_up"}, {w_down, "w_down"}, {dx, "dx"},
                        {dw_gate, "dw_gate"}, {dw_up, "dw_up"}, {dw_down, "dw_down"}},
                       16)) != MOE_OK)
    return st;
  if ((st = check_ptrs({{dlogits, "dlogits"}}, 4)) != MOE_OK) return st;
  if ((st = check_ptrs({{saved, "saved"}, {ws, "ws"}}, 256)) != MOE_OK) return st;
  if ((st = check_stream(stream)) != MOE_OK) return st;
  const Layout L = make_layout(*d);
  if (ws_bytes < L.bwd_total) return fail(MOE_ERR_WORKSPACE_TOO_SMALL, "backward workspace too small");
  const char* sv = static_cast<const char*>(saved);
  char* w = static_cast<char*>(ws);
  BwdParams p{};
  p.dy = dy;
  p.x = x;
  p.wg = w_gate;
  p.wu = w_up;
  p.wd = w_down;
  p.idx = reinterpret_cast<const int*>(sv + L.idx);
  p.weight = reinterpret_cast<const float*>(sv + L.weight);
  p.perm = reinterpret_cast<const int*>(sv + L.perm);
  p.ptok = reinterpret_cast<const int*>(sv + L.ptok);
  p.offsets = reinterpret_cast<const int*>(sv + L.offsets);
  p.pair_pos = reinterpret_cast<const int*>(sv + L.pair_pos);
  p.mtile = reinterpret_cast<const int2*>(sv + L.mtile);
  p.num_mtiles = reinterpret_cast<const int*>(sv + L.num_mtiles);
  p.mtile2 = reinterpret_cast<const int2*>(sv + L.mtile2);
  p.num_mtiles2 = reinterpret_cast<const int*>(sv + L.num_mtiles2);
  p.zeros = sv + L.zeros;
  p.qoff = reinterpret_cast<const int*>(sv + L.qoff);
  p.qc = L.qc;
  p.ab = sv + L.ab;
  p.hw = sv + L.hw;
  p.hwt = sv + L.hwt;
  p.dabt = w + L.dabt;
  p.dab = w + L.dab;
  p.gpart = reinterpret_cast<float*>(w + L.gpart);
  p.sched = reinterpret_cast<int*>(w + L.sched_b);
  p.dxp = w + L.dxp;
  p.dx = dx;
  p.dlogits = dlogits;
  p.dwg = dw_gate;
  p.dwu = dw_up;
  p.dwd = dw_down;
  p.T = d->T;
  p.rows = L.rows;
  p.H = d->H;
  p.F = d->F;
  p.k = d->topk;
  p.E = d->E_total;
  p.El = d->E_local;
  p.np = L.np;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (L.rc && (e = recompute_activations(*d, L, p, w, s)) != hipSuccess) return hip_fail(e, "recompute launch");
  if (L.mx) {
    // every backward GEMM operand as MXFP8 along its contraction axis; da and db are quantised in
    // the dH epilogue. MXFP8: the weights' backward orientation comes from the forward (`saved`);
    // FP8_BWD quantises it here, and with activation checkpointing the recompute did.
    auto u8 = [&](size_t o) { return reinterpret_cast<uint8_t*>(w + o); };
    const int El = d->E_local, H = d->H, F = d->F;
    const bool f8b = d->mode == MOE_MODE_FP8_BWD, blk = d->mode == MOE_MODE_FP8;
    const bool wq_here = f8b || L.rc;
    const uint8_t* wdtq = wq_here ? u8(L.wdtq) : reinterpret_cast<const uint8_t*>(sv + L.sv_wdtq);
    const uint8_t* wdts = wq_here ? u8(L.wdts) : reinterpret_cast<const uint8_t*>(sv + L.sv_wdts);
    const uint8_t* wgutq = wq_here ? u8(L.wgutq) : reinterpret_cast<const uint8_t*>(sv + L.sv_wgutq);
    const uint8_t* wguts = wq_here ? u8(L.wguts) : reinterpret_cast<const uint8_t*>(sv + L.sv_wguts);
    if (f8b &&
        ((e = launch_quant_cols(w_down, u8(L.wdtq), u8(L.wdts), El, H, F, H, 0, "mx_quant_w_down_t", s)) != hipSuccess ||
         (e = launch_quant_cols(w_gate, u8(L.wgutq), u8(L.wguts), El, F, H, 2 * F, 0, "mx_quant_w_gate_t", s)) != hipSuccess ||
         (e = launch_quant_cols(w_up, u8(L.wgutq), u8(L.wguts), El, F, H, 2 * F, F, "mx_quant_w_up_t", s)) != hipSuccess))
      return hip_fail(e, "quantise launch");
    if ((e = launch_quant_rows(dy, u8(L.dyq), u8(L.dys), d->T * d->H, "mx_quant_dy", s, blk)) != hipSuccess ||
        (e = launch_gather_t_quant(dy, p.ptok, p.offsets, p.qoff, El, H, L.qc, u8(L.dytq), u8(L.dyts), "mx_quant_dy_t",
                                   s, blk)) != hipSuccess ||
        (e = launch_gather_t_quant(x, p.ptok, p.offsets, p.qoff, El, H, L.qc, u8(L.xtq), u8(L.xts), "mx_quant_x_t",
                                   s, blk)) != hipSuccess)
      return hip_fail(e, "quantise launch");
    p.blk = blk;
    p.dyq = u8(L.dyq);
    p.dys = u8(L.dys);
    p.wdtq = wdtq;
    p.wdts = wdts;
    p.wgutq = wgutq;
    p.wguts = wguts;
    p.dytq = u8(L.dytq);
    p.dyts = u8(L.dyts);
    p.xtq = u8(L.xtq);
    p.xts = u8(L.xts);
    p.hwtq = reinterpret_cast<const uint8_t*>(L.rc ? w + L.r_hwt : sv + L.hwt);
    p.hwts = reinterpret_cast<const uint8_t*>(L.rc ? w + L.r_hwts : sv + L.hwts);
    p.dabq = u8(L.dabq);
    p.dabs = u8(L.dabs);
    p.dabtq = u8(L.dabtq);
    p.dabts = u8(L.dabts);
    e = launch_backward_gemms_mx(p, persistent_grid(1), s);
  } else {
    e = d->mode == MOE_MODE_FP32 ? launch_backward<float>(p, persistent_grid(2), s)
                                 : launch_backward_gemms_bf16(p, persistent_grid(1), s);
  }
  if (e != hipSuccess) {
    side_stream_join(s);   // whatever reached the side stream is still waited for
    return hip_fail(e, "backward GEMM launch");
  }
  e = d->mode == MOE_MODE_FP32 ? launch_combine_bwd<float>(p, s) : launch_combine_bwd<bf16>(p, s);
  hipError_t ej = side_stream_join(s);
  if (e != hipSuccess) return hip_fail(e, "backward combine launch");
  if (ej != hipSuccess) return hip_fail(ej, "side stream join");
  return MOE_OK;
}

// ------------------------------------------------------------------------------------------------
// Router projection in front of the layer

namespace {
struct RouterLayout {
  int Ep;          // E_total rounded up to 64 (the bf16 copy of dlogits and the partial rows)
  int Sf, kcf;     // forward: H split Sf ways, kcf elements each
  int Sb, kcb;     // dW_r: T split Sb ways, kcb tokens each (a multiple of 64)
  size_t fwd_part, fwd_total;
  size_t bwd_zero, bwd_dlb, bwd_part, bwd_total;
};

RouterLayout router_layout(const moe_desc& d) {
  RouterLayout R{};
  const int64_t T = d.T;
  const int64_t H = d.H, E = d.E_total;
  R.Ep = (int)((E + 63) / 64 * 64);
  const int64_t mtn = (T + 255) / 256, etn = (E + 255) / 256, htn = H / 256;
  // about one 256x256 tile per CU or more: split H (S in {1, 2, 4}; H is a multiple of 256)
  R.Sf = 1;
  while (R.Sf < 4 && mtn * etn * R.Sf * 2 <= 256) R.Sf *= 2;
  R.kcf = (int)(H / R.Sf);
  const int64_t want = std::max<int64_t>(1, 256 / (etn * htn));
  R.kcb = (int)(((T + want - 1) / want + 63) / 64 * 64);
  R.Sb = (int)((T + R.kcb - 1) / R.kcb);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = align256(off + bytes);
    return at;
  };
  const bool f32 = d.mode == MOE_MODE_FP32;   // the fp32 test mode's kernels need no workspace
  R.fwd_part = take(f32 ? 0 : (size_t)R.Sf * T * R.Ep * 4);
  R.fwd_total = std::max<size_t>(off, 256);
  off = 0;
  R.bwd_zero = take(f32 ? 0 : kZeroBytes);
  R.bwd_dlb = take(f32 ? 0 : (size_t)T * R.Ep * 2);
  R.bwd_part = take(f32 ? 0 : (size_t)R.Sb * E * H * 4);
  R.bwd_total = std::max<size_t>(off, 256);
  return R;
}

moe_status router_checks(const moe_desc* d) { return validate(d); }
}  // namespace

moe_status moe_query_router_sizes(const moe_desc* d, size_t* fwd_ws, size_t* bwd_ws) {
  g_last_error.clear();
  moe_status st = router_checks(d);
  if (st != MOE_OK) return st;
  const RouterLayout R = router_layout(*d);
  if (fwd_ws) *fwd_ws = R.fwd_total;
  if (bwd_ws) *bwd_ws = R.bwd_total;
  return MOE_OK;
}

moe_status moe_router_fwd(const moe_desc* d, const void* x, const void* w_router, float* logits, void* ws,
                          size_t ws_bytes, void* stream) {
  g_last_error.clear();
  moe_status st = router_checks(d);
  if (st != MOE_OK) return st;
  if ((st = check_ptrs({{x, "x"}, {w_router, "w_router"}, {logits, "logits"}}, 16)) != MOE_OK) return st;
  if ((st = check_ptrs({{ws, "ws"}}, 256)) != MOE_OK) return st;
  if ((st = check_stream(stream)) != MOE_OK) return st;
  const RouterLayout R = router_layout(*d);
  if (ws_bytes < R.fwd_total) return fail(MOE_ERR_WORKSPACE_TOO_SMALL, "router forward workspace too small");
  RouterParams p{};
  p.x = x;
  p.wr = w_router;
  p.part = reinterpret_cast<float*>(static_cast<char*>(ws) + R.fwd_part);
  p.logits = logits;
  p.T = d->T;
  p.H = d->H;
  p.E = d->E_total;
  p.Ep = R.Ep;
  p.S = R.Sf;
  p.kc = R.kcf;
  // up to 256 experts: the fused forward's projection (one workgroup per 64 tokens, all experts, no
  // partial sums), so that these logits are bitwise the ones moe_fwd_router routes on
  hipError_t e = d->mode == MOE_MODE_FP32 ? launch_router_fwd_f32(p, static_cast<hipStream_t>(stream))
                 : d->E_total <= 256
                     ? launch_router_logits_bf16(x, w_router, logits, d->T, d->H, d->E_total,
                                                 static_cast<hipStream_t>(stream))
                     : launch_router_fwd_bf16(p, persistent_grid(1), static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "router forward launch");
  return MOE_OK;
}

moe_status moe_router_bwd(const moe_desc* d, const void* x, const void* w_router, const float* dlogits, void* dx,
                          void* dw_router, void* ws, size_t ws_bytes, void* stream) {
  g_last_error.clear();
  moe_status st = router_checks(d);
  if (st != MOE_OK) return st;
  if ((st = check_ptrs({{x, "x"}, {w_router, "w_router"}, {dx, "dx"}, {dw_router, "dw_router"}}, 16)) != MOE_OK)
    return st;
  if ((st = check_ptrs({{dlogits, "dlogits"}}, 4)) != MOE_OK) return st;
  if ((st = check_ptrs({{ws, "ws"}}, 256)) != MOE_OK) return st;
  if ((st = check_stream(stream)) != MOE_OK) return st;
  const RouterLayout R = router_layout(*d);
  if (ws_bytes < R.bwd_total) return fail(MOE_ERR_WORKSPACE_TOO_SMALL, "router backward workspace too small");
  char* w = static_cast<char*>(ws);
  RouterParams p{};
  p.x = x;
  p.wr = w_router;
  p.part = reinterpret_cast<float*>(w + R.bwd_part);
  p.dlogits = dlogits;
  p.dlb = w + R.bwd_dlb;
  p.dx = dx;
  p.dwr = dw_router;
  p.zeros = w + R.bwd_zero;
  p.T = d->T;
  p.H = d->H;
  p.E = d->E_total;
  p.Ep = R.Ep;
  p.S = R.Sb;
  p.kc = R.kcb;
  hipError_t e = d->mode == MOE_MODE_FP32 ? launch_router_bwd_f32(p, static_cast<hipStream_t>(stream))
                                          : launch_router_bwd_bf16(p, persistent_grid(1), static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "router backward launch");
  return MOE_OK;
}

moe_status moe_mx_quantize(const void* in, int64_t rows, int64_t cols, int axis, uint8_t* q, uint8_t* scales,
                           void* stream) {
  g_last_error.clear();
  moe_status st;
  if ((st = check_ptrs({{in, "in"}, {q, "q"}}, 16)) != MOE_OK) return st;
  if ((st = check_ptrs({{scales, "scales"}}, 4)) != MOE_OK) return st;
  if ((st = check_stream(stream)) != MOE_OK) return st;
  if (rows < 1 || cols < 1) return fail(MOE_ERR_INVALID_ARG, "rows and cols must be positive");
  if (axis != 0 && axis != 1) return fail(MOE_ERR_INVALID_ARG, "axis must be 0 or 1");
  if (axis == 1 && cols % 32 != 0) return fail(MOE_ERR_UNSUPPORTED_SHAPE, "cols must be a multiple of 32 (axis 1)");
  if (axis == 0 && (rows % 128 != 0 || cols % 64 != 0))
    return fail(MOE_ERR_UNSUPPORTED_SHAPE, "rows must be a multiple of 128 and cols of 64 (axis 0)");
  if (rows * cols >= (int64_t(1) << 34)) return fail(MOE_ERR_UNSUPPORTED_SHAPE, "rows*cols must be < 2^34");
  if (axis == 0 && (rows / 128 > 65535 || cols / 64 > INT32_MAX))
    return fail(MOE_ERR_UNSUPPORTED_SHAPE, "matrix too large for axis 0");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t e = axis == 1 ? launch_quant_rows(in, q, scales, rows * cols, "mx_quant_rows", s)
                                 : launch_quant_cols(in, q, scales, 1, (int)rows, (int)cols, rows, 0, "mx_quant_cols", s);
  if (e != hipSuccess) return hip_fail(e, "quantise launch");
  return MOE_OK;
}

moe_status moe_fp8_block_quantize(const void* in, int64_t rows, int64_t cols, int weight, uint8_t* q,
                                  uint8_t* scales, uint8_t* qt, uint8_t* scales_t, void* stream) {
  g_last_error.clear();
  moe_status st;
  if ((st = check_ptrs({{in, "in"}, {q, "q"}}, 16)) != MOE_OK) return st;
  if ((st = check_ptrs({{scales, "scales"}}, 4)) != MOE_OK) return st;
  if ((st = check_stream(stream)) != MOE_OK) return st;
  if (rows < 1 || cols < 1) return fail(MOE_ERR_INVALID_ARG, "rows and cols must be positive");
  if (weight != 0 && weight != 1) return fail(MOE_ERR_INVALID_ARG, "weight must be 0 or 1");
  if (weight == 1) {
    if ((st = check_ptrs({{qt, "qt"}}, 16)) != MOE_OK) return st;
    if ((st = check_ptrs({{scales_t, "scales_t"}}, 4)) != MOE_OK) return st;
    if (rows % 128 != 0) return fail(MOE_ERR_UNSUPPORTED_SHAPE, "rows must be a multiple of 128 (weight)");
    if (rows / 128 > 65535) return fail(MOE_ERR_UNSUPPORTED_SHAPE, "matrix too large for the weight form");
  }
  if (cols % 128 != 0) return fail(MOE_ERR_UNSUPPORTED_SHAPE, "cols must be a multiple of 128");
  if (rows * cols >= (int64_t(1) << 34)) return fail(MOE_ERR_UNSUPPORTED_SHAPE, "rows*cols must be < 2^34");
  if (cols > INT32_MAX || rows > INT32_MAX) return fail(MOE_ERR_UNSUPPORTED_SHAPE, "matrix too large");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t e =
      weight == 0 ? launch_quant_rows(in, q, scales, rows * cols, "fp8b_quant_rows", s, true)
                  : launch_quant_both(in, q, scales, qt, scales_t, 1, (int)rows, (int)cols, rows, 0, "fp8b_quant_weight",
                                      s, true);
  if (e != hipSuccess) return hip_fail(e, "quantise launch");
  return MOE_OK;
}

moe_status moe_profile_enable(int max_launches) {
  g_last_error.clear();
  if (max_launches < 1) return fail(MOE_ERR_INVALID_ARG, "max_launches must be >= 1");
  Prof& P = prof();
  std::lock_guard<std::mutex> g(P.mu);
  while ((int)P.ev.size() < 2 * max_launches) {
    hipEvent_t ev;
    hipError_t e = hipEventCreate(&ev);
    if (e != hipSuccess) return hip_fail(e, "hipEventCreate");
    P.ev.push_back(ev);
  }
  P.cap = max_launches;
  P.rec_kernel.assign(max_launches, -1);
  P.n = 0;
  P.names.clear();
  P.launches.clear();
  P.total_ms.clear();
  P.on = true;
  return MOE_OK;
}

moe_status moe_profile_disable(void) {
  Prof& P = prof();
  std::lock_guard<std::mutex> g(P.mu);
  P.on = false;
  return MOE_OK;
}

moe_status moe_profile_collect(void) {
  g_last_error.clear();
  Prof& P = prof();
  std::lock_guard<std::mutex> g(P.mu);
  for (int i = 0; i < P.n; ++i) {
    hipError_t e = hipEventSynchronize(P.ev[2 * i + 1]);
    if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize");
    float ms = 0.f;
    e = hipEventElapsedTime(&ms, P.ev[2 * i], P.ev[2 * i + 1]);
    if (e != hipSuccess) return hip_fail(e, "hipEventElapsedTime");
    const int kid = P.rec_kernel[i];
    P.launches[kid] += 1;
    P.total_ms[kid] += ms;
  }
  P.n = 0;
  return MOE_OK;
}

moe_status moe_profile_kernel(int i, const char** name, int* launches, double* total_ms) {
  Prof& P = prof();
  std::lock_guard<std::mutex> g(P.mu);
  if (i < 0 || i >= (int)P.names.size()) return MOE_ERR_INVALID_ARG;
  if (name) *name = P.names[i].c_str();
  if (launches) *launches = P.launches[i];
  if (total_ms) *total_ms = P.total_ms[i];
  return MOE_OK;
}

}  // extern "C"
