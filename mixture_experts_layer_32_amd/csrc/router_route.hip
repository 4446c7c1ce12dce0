// The router projection fused with the routing: logits = x W_r^T on the bf16 MFMA, top-k of the
// logits, renormalised softmax weights and the per-block expert masks, in one kernel; the caller's
// logits are written as a by-product. The pages fold the routing into the fused operation ("Prime
// Mega MoE: kernel fuso per l'addestramento MoE" on "Prime Mega MoE: il kernel che accelera il
// training AI del 55%"); the projection is read as the usual linear router without bias.
//
// A block takes 64 tokens (one routing block: its masks are one 64-bit word per expert) and all of
// the experts (E <= 128 NB). Its 8 wavefronts split them as 2 token halves x 4 expert groups: each
// owns 32 tokens x 32 NB experts, NB blocks of v_mfma_f32_32x32x16_bf16 with fp32 accumulation over
// H. The operands reach LDS by direct-to-LDS loads through a ring of S stages of RB bytes of
// contraction per row (RB / 2 elements), one barrier per stage: after it, the stage read in the
// previous step is refilled with the stage S - 1 ahead. The x rows stream from HBM once; W_r (0.5 MB
// at E = 128, H = 2048) stays in L2. A stage carries little arithmetic per wave (RB / 32 MFMA steps
// of NB blocks), so even and odd steps accumulate into two sets of registers (two dependency chains
// instead of one), added at the end, and the fragments of the next step are read while the current
// one multiplies. At the 30B-A3B shape this takes 32 us (22 us without the top-k), against 36 us for
// the first form of the kernel (128-byte-deep stages with two barriers each and one chain).
#include "engine.h"
#include "moe_internal.h"
#include "route_device.h"

namespace moe {
namespace {

using namespace eng;

constexpr int RT = kRouteTokens;   // tokens per block

// wait until at most n stages of NL loads each are in flight (n <= N, a run-time value)
template <int NL, int N>
__device__ __forceinline__ void wait_ktiles(int n) {
  if constexpr (N == 0) {
    wait_vm<0>();
  } else {
    if (n >= N) wait_vm<N * NL>();
    else wait_ktiles<NL, N - 1>(n);
  }
}

// RB-byte rows of a stage: 16-byte chunk c of row r at slot c ^ swz(r), so that a ds_read_b128 of 16
// consecutive rows at one chunk touches all 64 banks once
template <int RB>
__device__ __forceinline__ int rswz(int r) { return RB == 256 ? (r & 15) : ((r >> 1) & 7); }
template <int RB>
__device__ __forceinline__ const char* rat(const char* tile, int r, int c) {
  return tile + r * RB + ((c ^ rswz<RB>(r)) << 4);
}

// TOPK: route the block's tokens (top-k, weights, masks) after writing the logits; without it the
// kernel is the projection alone (moe_router_fwd), whose logits are then bitwise those the routing
// uses in the fused forward.
template <int NB, int RB, int S, bool TOPK>
__global__ __launch_bounds__(512, 1) void k_router_topk_bf16(RouteParams rp, const bf16* __restrict__ x,
                                                             const bf16* __restrict__ wr, float* __restrict__ lg_out,
                                                             int H) {
  constexpr int NE = 128 * NB;                  // expert rows per stage (W_r rows past E are clamped)
  constexpr int KS = RB / 32;                   // 16-deep MFMA steps per stage
  constexpr int NC = RB / 16;                   // 16-byte chunks per row
  constexpr int RPI = 64 / NC;                  // rows per wave instruction (1 KB)
  constexpr int LX = RT / (8 * RPI), LW = NE / (8 * RPI);   // x and W_r loads per lane per stage
  constexpr int NL = LX + LW;
  constexpr int XB = RT * RB, STB = XB + NE * RB;
  constexpr int LDL = NE + 4;                   // staged logits row stride (floats): 4 banks mod 64
  static_assert(KS % 2 == 0 && LX >= 1 && LW >= 1, "stage geometry");
  static_assert(RT * LDL * 4 <= S * STB, "the logits fit the ring");
  static_assert(S * STB + kMaxExperts * 8 <= 160 * 1024, "LDS");
  __shared__ __attribute__((aligned(1024))) char smem[S * STB];
  __shared__ unsigned long long mask[kMaxExperts];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, th = w >> 2, eg = w & 3;
  const int64_t t0 = (int64_t)blockIdx.x * RT;
  const int E = rp.E;
  if (TOPK)
    for (int e = tid; e < rp.El; e += 512) mask[e] = 0ull;
  // Load i of this lane moves row (w L + i) RPI + lane / NC of its operand, chunk slot lane % NC
  // (global chunk slot ^ swizzle): one wave instruction fills 1 KB of whole row segments.
  const char* xp[LX];
  const char* wp[LW];
#pragma unroll
  for (int i = 0; i < LX; ++i) {
    const int r = (w * LX + i) * RPI + lane / NC;
    const int64_t tok = min(t0 + r, rp.T - 1);   // rows past T feed discarded outputs
    xp[i] = reinterpret_cast<const char*>(x + tok * H) + 16 * ((lane % NC) ^ rswz<RB>(r));
  }
#pragma unroll
  for (int i = 0; i < LW; ++i) {
    const int r = (w * LW + i) * RPI + lane / NC;
    const int e = min(r, E - 1);                 // rows past E feed discarded outputs
    wp[i] = reinterpret_cast<const char*>(wr + (size_t)e * H) + 16 * ((lane % NC) ^ rswz<RB>(r));
  }
  auto issue = [&](int kt, char* st) {
#pragma unroll
    for (int i = 0; i < LX; ++i) gl2lds(xp[i] + (size_t)kt * RB, st + (w * LX + i) * 1024);
#pragma unroll
    for (int i = 0; i < LW; ++i) gl2lds(wp[i] + (size_t)kt * RB, st + XB + (w * LW + i) * 1024);
  };
  f32x16 acc[NB], acc2[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j)
#pragma unroll
    for (int q = 0; q < 16; ++q) acc[j][q] = acc2[j][q] = 0.f;
  const int arow = 32 * th + (lane & 31), brow = 32 * NB * eg + (lane & 31);
  auto frags = [&](const char* st, int ks, bf16x8& fa, bf16x8 (&fb)[NB]) {
    fa = *reinterpret_cast<const bf16x8*>(rat<RB>(st, arow, 2 * ks + (lane >> 5)));
#pragma unroll
    for (int j = 0; j < NB; ++j)
      fb[j] = *reinterpret_cast<const bf16x8*>(rat<RB>(st + XB, brow + 32 * j, 2 * ks + (lane >> 5)));
  };
  const int nk = 2 * H / RB;
#pragma unroll
  for (int q = 0; q < S - 1; ++q)
    if (q < nk) issue(q, smem + q * STB);
  for (int kt = 0; kt < nk; ++kt) {
    wait_ktiles<NL, S - 2>(min(S - 2, nk - 1 - kt));   // stage kt has landed; the later ones may not
    block_sync();   // publishes stage kt; every wave is done reading stage kt - 1
    if (kt + S - 1 < nk) issue(kt + S - 1, smem + ((kt + S - 1) % S) * STB);
    const char* st = smem + (kt % S) * STB;
    bf16x8 fa0, fb0[NB], fa1, fb1[NB];
    frags(st, 0, fa0, fb0);
#pragma unroll
    for (int ks = 0; ks < KS; ks += 2) {
      frags(st, ks + 1, fa1, fb1);   // the next step's fragments while this step multiplies
#pragma unroll
      for (int j = 0; j < NB; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb0[j], fa0, acc[j], 0, 0, 0);
      if (ks + 2 < KS) frags(st, ks + 2, fa0, fb0);
#pragma unroll
      for (int j = 0; j < NB; ++j) acc2[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb1[j], fa1, acc2[j], 0, 0, 0);
    }
  }
  block_sync();   // every wave is done with the ring
  // logits to LDS: accumulator element 4a + b of block j is token 32 th + (lane & 31), expert
  // 32 NB eg + 32 j + 8a + 4(lane >> 5) + b
  float* lg = reinterpret_cast<float*>(smem);
#pragma unroll
  for (int j = 0; j < NB; ++j)
#pragma unroll
    for (int a = 0; a < 4; ++a)
      *reinterpret_cast<float4*>(lg + arow * LDL + 32 * NB * eg + 32 * j + acc_n(a, lane)) =
          make_float4(acc[j][4 * a] + acc2[j][4 * a], acc[j][4 * a + 1] + acc2[j][4 * a + 1],
                      acc[j][4 * a + 2] + acc2[j][4 * a + 2], acc[j][4 * a + 3] + acc2[j][4 * a + 3]);
  __syncthreads();
  // the caller's logits [T, E]: the block's rows are contiguous; a wave per row, 16-byte stores when
  // the rows are 16-byte aligned
  const int nrow = (int)min((int64_t)RT, rp.T - t0);
  float* lo = lg_out + t0 * E;
  if ((E & 3) == 0 && (reinterpret_cast<uintptr_t>(lg_out) & 15) == 0) {
    for (int r = w; r < nrow; r += 8)
      for (int c = 4 * lane; c < E; c += 256)
        *reinterpret_cast<float4*>(lo + (size_t)r * E + c) = *reinterpret_cast<const float4*>(lg + r * LDL + c);
  } else {
    for (int r = w; r < nrow; r += 8)
      for (int c = lane; c < E; c += 64) lo[(size_t)r * E + c] = lg[r * LDL + c];
  }
  if constexpr (!TOPK) return;
  // top-k: 8 lanes per token
  const int tl = tid >> 3;
  if (t0 + tl < rp.T)
    route_token<8, 8>(rp, t0 + tl, tl, tid & 7, [&](int e) { return lg[tl * LDL + e]; }, mask);
  __syncthreads();
  for (int e = tid; e < rp.El; e += 512) {
    const size_t qq = (size_t)blockIdx.x * rp.El + e;
    rp.blk_mask[qq] = mask[e];
    rp.blk_count[qq] = __popcll(mask[e]);
  }
}

}  // namespace

hipError_t launch_router_route_bf16(const RouteParams& p, const void* x, const void* w_router, float* logits, int H,
                                    hipStream_t s) {
  prof_mark_begin("router_topk_fused", s);
  const bf16* xb = static_cast<const bf16*>(x);
  const bf16* wb = static_cast<const bf16*>(w_router);
  if (p.E <= 128) k_router_topk_bf16<1, 256, 3, true><<<p.nblk, 512, 0, s>>>(p, xb, wb, logits, H);
  else k_router_topk_bf16<2, 128, 3, true><<<p.nblk, 512, 0, s>>>(p, xb, wb, logits, H);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  prof_mark_end(s);
  return launch_route_tail(p, s);
}

hipError_t launch_router_logits_bf16(const void* x, const void* w_router, float* logits, int64_t T, int H, int E,
                                     hipStream_t s) {
  RouteParams p{};   // the projection reads only T and E
  p.T = T;
  p.E = E;
  const unsigned nblk = (unsigned)((T + kRouteTokens - 1) / kRouteTokens);
  prof_mark_begin("router_fwd_gemm", s);
  const bf16* xb = static_cast<const bf16*>(x);
  const bf16* wb = static_cast<const bf16*>(w_router);
  if (E <= 128) k_router_topk_bf16<1, 256, 3, false><<<nblk, 512, 0, s>>>(p, xb, wb, logits, H);
  else k_router_topk_bf16<2, 128, 3, false><<<nblk, 512, 0, s>>>(p, xb, wb, logits, H);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  prof_mark_end(s);
  return hipSuccess;
}

}  // namespace moe
