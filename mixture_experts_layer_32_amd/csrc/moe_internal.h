// Host-side internals of libmoe: buffer layout and kernel launchers.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/moe.h"

namespace moe {

constexpr int kBM = 128;            // rows per M-tile of the fp32 row-tiled grouped GEMMs
constexpr int kBM2 = 256;           // rows per M-tile of the bf16 row-tiled grouped GEMMs
constexpr int kZeroBytes = 1024;    // zero page read by the bf16 GEMMs for out-of-range rows
constexpr int kRouteTokens = 64;    // tokens per routing block (one 64-bit mask word per expert)
constexpr int kMaxExperts = 512;
constexpr int kMaxTopk = 32;
constexpr int kSchedInts = 16;      // ints per GEMM's tile-scheduler slot (8 per-XCD counters, padded to 64 B)
constexpr int kSchedSlots = 8;      // scheduler slots per workspace
// backward slots holding the weight-gradient GEMMs' per-XCD tile ranges (9 boundaries each)
constexpr int kSchedWgradDown = 2, kSchedWgradGateup = 3;

// Byte offsets of every region inside the three caller-provided buffers.
struct Layout {
  int64_t rows;        // T*k: upper bound on routed pairs
  int nblk_route;      // ceil(T / kRouteTokens)
  int mtile_cap;       // upper bound on 128-row M-tiles: rows / kBM + E_local + 1
  int mtile2_cap;      // upper bound on 256-row M-tiles
  int np;              // partial sums of g per pair: F / 64 (fp32), 4*ceil(F/256) (bf16), 2*ceil(F/256) (fp8)
  size_t elem;         // bytes per stored element (4 or 2)
  int qpad;            // pair-contiguous segments are padded to a multiple of qpad pairs (32, or 64 in MX modes)
  bool mx;             // MXFP8 or FP8_BWD
  bool rc;             // activation checkpointing: the backward recomputes the gate/up activations
  // saved
  int64_t qc;          // row stride of the pair-contiguous transposed copies (bf16 and fp8 engines)
  size_t idx, weight, counts, offsets, perm, ptok, pair_pos, mtile, num_mtiles, mtile2, num_mtiles2, zeros, qoff, ab, hw,
      hwt, hwts, saved_total;
  // MXFP8: the weights quantised along their other axis by the forward, for the backward (in
  // saved); FP8_BWD: the backward quantises them into its workspace (wdtq.. below)
  size_t sv_wdtq, sv_wdts, sv_wgutq, sv_wguts;
  // forward workspace (MXFP8: quantised operands; BF16 and FP8_BWD: the bf16 hw)
  size_t sched_f, blk_mask, blk_count, blk_prefix, o, xq, xs, wgq, wgs, wuq, wus, wdq, wds, hwq, hws, hw16, fwd_total;
  // backward workspace (MX: quantised operands)
  size_t sched_b, dab, gpart, dxp, dabt, dyq, dys, wdtq, wdts, wgutq, wguts, dytq, dyts, xtq, xts, dabq, dabs, dabtq, dabts;
  // activation checkpointing: the forward's scratch for the fp32 engine's a, b and hw (the forward
  // workspace), and the backward's recomputed activations and quantised forward operands
  size_t f_ab, f_hw, r_sched, r_ab, r_hw, r_hwt, r_hwts, r_xq, r_xs, r_wgq, r_wgs, r_wuq, r_wus, bwd_total;
};

Layout make_layout(const moe_desc& d);

// Launch helper: optional event timing, error capture.
void prof_mark_begin(const char* name, hipStream_t s);
void prof_mark_end(hipStream_t s);

struct RouteParams {
  const float* logits;
  int* idx;
  float* weight;
  int* counts;
  int* offsets;
  int* perm;
  int* ptok;
  int* pair_pos;
  int2* mtile;
  int* num_mtiles;
  int2* mtile2;
  int* num_mtiles2;
  uint4* zeros;
  int* qoff;
  unsigned long long* blk_mask;
  int* blk_count;
  int* blk_prefix;
  int* sched;          // the forward GEMMs' tile-scheduler counters, zeroed by the routing
  int64_t T;
  int E, El, e0, k, nblk, qpad;
};
hipError_t launch_route(const RouteParams& p, hipStream_t s);
// the routing after the top-k (its per-block masks and counts in place): scans, offsets, permutation
hipError_t launch_route_tail(const RouteParams& p, hipStream_t s);
// the router projection fused with the top-k (bf16 x and W_r, E <= 256, k <= 8), then the routing
// tail; the logits [T, E] fp32 are written to `logits`
hipError_t launch_router_route_bf16(const RouteParams& p, const void* x, const void* w_router, float* logits, int H,
                                    hipStream_t s);
// the projection of launch_router_route_bf16 alone (E <= 256): logits [T, E] fp32
hipError_t launch_router_logits_bf16(const void* x, const void* w_router, float* logits, int64_t T, int H, int E,
                                     hipStream_t s);

// Row-tiled grouped GEMMs and wgrad GEMMs; T = float or bf16.
struct FwdParams {
  const void* x;
  const void* wg;
  const void* wu;
  const void* wd;
  const int* perm;
  const int* ptok;
  const int* offsets;
  const int2* mtile;
  const int* num_mtiles;
  const int2* mtile2;
  const int* num_mtiles2;
  const void* zeros;
  const int* qoff;
  int64_t qc;
  const float* weight;
  void* ab;
  void* hw;
  void* hwt;
  void* o;
  const int* pair_pos;
  void* y;
  // MXFP8 operands: E4M3 bytes and e8m0 scales ([rows][K/32]), all K-major
  const uint8_t *xq, *xs, *wgq, *wgs, *wuq, *wus, *wdq, *wds;
  uint8_t *hwq, *hws, *hwtq, *hwts;
  bool blk;            // blockwise FP8 scales instead of MXFP8 (fp8 engine only)
  int* sched;          // tile-scheduler counters (kSchedSlots slots), zero at launch
  int64_t T;
  int H, F, k, El;
};
template <class T> hipError_t launch_forward_gemms(const FwdParams& p, int grid, hipStream_t s, bool recompute = false);
// tpw: tokens per wavefront (combine_tpw)
template <class T> hipError_t launch_combine(const void* src, const int* pair_pos, void* out, int64_t ntok,
                                             int k, int H, int tpw, hipStream_t s);

struct BwdParams {
  const void* dy;
  const void* x;
  const void* wg;
  const void* wu;
  const void* wd;
  const int* idx;
  const float* weight;
  const int* perm;
  const int* ptok;
  const int* offsets;
  const int* pair_pos;
  const int2* mtile;
  const int* num_mtiles;
  const int2* mtile2;
  const int* num_mtiles2;
  const void* zeros;
  const int* qoff;
  int64_t qc;
  const void* ab;
  const void* hw;
  const void* hwt;
  void* dab;
  void* dabt;
  float* gpart;
  void* dxp;
  void* dx;
  float* dlogits;
  void* dwg;
  void* dwu;
  void* dwd;
  // MXFP8 operands: E4M3 bytes and e8m0 scales ([rows][K/32]), all K-major
  const uint8_t *dyq, *dys, *wdtq, *wdts, *wgutq, *wguts, *dytq, *dyts, *xtq, *xts, *hwtq, *hwts;
  uint8_t *dabq, *dabs, *dabtq, *dabts;
  bool blk;            // blockwise FP8 scales instead of MXFP8 (fp8 engine only)
  int* sched;          // tile-scheduler counters (kSchedSlots slots), zeroed before the GEMMs
  int64_t T, rows;
  int H, F, k, E, El, np;
};
template <class T> hipError_t launch_backward(const BwdParams& p, int grid, hipStream_t s);
template <class T> hipError_t launch_combine_bwd(const BwdParams& p, hipStream_t s);
// gate/up and down GEMMs; recompute: the gate/up GEMM alone, as the backward's recompute under
// activation checkpointing (bf16: with its tile counters at p.sched zeroed first)
hipError_t launch_forward_gemms_bf16(const FwdParams& p, int grid, hipStream_t s, bool recompute = false);
hipError_t launch_backward_gemms_bf16(const BwdParams& p, int grid, hipStream_t s);
// zeroes the backward's tile counters and splits the weight-gradient tile lists over the XCDs by
// cost (ktile: pairs per K-tile of the engine)
hipError_t launch_sched_setup(const BwdParams& p, int ktile, hipStream_t s);

// Router projection in front of the layer (bf16 engine): logits = x W_r^T; backward dW_r and the
// router's part of dx. The GEMMs with a long contraction split it S ways (kc elements per split)
// and add the fp32 partial sums in a fixed order.
struct RouterParams {
  const void* x;         // [T, H] bf16 (fp32 in the fp32 test mode, likewise wr, dx, dwr)
  const void* wr;        // [E, H] bf16
  float* part;           // split partial sums: [S][T][Ep] (forward), [S][E][H] (backward)
  float* logits;         // [T, E] fp32 (forward output)
  const float* dlogits;  // [T, E] fp32 (backward input)
  void* dlb;             // [T, Ep] bf16 copy of dlogits, zero-padded (backward)
  void* dx;              // [T, H] bf16, accumulated into (backward)
  void* dwr;             // [E, H] bf16 (backward output)
  void* zeros;           // zero page of kZeroBytes (backward)
  int64_t T;
  int H, E, Ep, S, kc;   // Ep = E rounded up to 64; S splits of kc elements of H (fwd) or T (bwd)
};
hipError_t launch_router_fwd_bf16(const RouterParams& p, int grid, hipStream_t s);
hipError_t launch_router_bwd_bf16(const RouterParams& p, int grid, hipStream_t s);
hipError_t launch_router_fwd_f32(const RouterParams& p, hipStream_t s);   // fp32 test mode
hipError_t launch_router_bwd_f32(const RouterParams& p, hipStream_t s);

hipError_t launch_forward_gemms_mx(const FwdParams& p, int grid, hipStream_t s, bool recompute = false);
hipError_t launch_backward_gemms_mx(const BwdParams& p, int grid, hipStream_t s);
hipError_t launch_quant_rows(const void* in, uint8_t* q, uint8_t* sc, int64_t n, const char* name, hipStream_t s,
                             bool blk = false);
hipError_t launch_quant_cols(const void* in, uint8_t* q, uint8_t* sc, int B, int R, int C, int64_t ldo, int col0,
                             const char* name, hipStream_t s);
hipError_t launch_quant_both(const void* in, uint8_t* qr, uint8_t* sr, uint8_t* qc, uint8_t* scc, int B, int R, int C,
                             int64_t ldo, int col0, const char* name, hipStream_t s, bool blk = false);
hipError_t launch_gather_t_quant(const void* x, const int* ptok, const int* offsets, const int* qoff, int El, int H,
                                 int64_t qc, uint8_t* q, uint8_t* sc, const char* name, hipStream_t s,
                                 bool blk = false);

int persistent_grid(int blocks_per_cu);
// The device's side stream for the backward's weight gradients (moe_api.hip). side_stream_fork
// orders it after the work on s so far and returns it (null: no side stream, run everything on s);
// from then until side_stream_join the calling thread holds the device's side-stream lock.
// side_stream_mark records a point on s, side_stream_wait_mark makes the side stream wait for it;
// side_stream_join, after the backward's last launch on s, makes s wait for the side stream's work
// and releases the lock (nothing if this thread did not fork). Every fork must be joined.
hipStream_t side_stream_fork(hipStream_t s);
hipError_t side_stream_mark(hipStream_t s);
hipError_t side_stream_wait_mark();
hipError_t side_stream_join(hipStream_t s);

}  // namespace moe
