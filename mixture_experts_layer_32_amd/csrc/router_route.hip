// The router projection fused with the routing: logits = x W_r^T on the bf16 MFMA, top-k of the
// logits, renormalised softmax weights and the per-block expert masks, in one kernel; the caller's
// logits are written as a by-product. The pages fold the routing into the fused operation ("Prime
// Mega MoE: kernel fuso per l'addestramento MoE" on "Prime Mega MoE: il kernel che accelera il
// training AI del 55%"); the projection is read as the usual linear router without bias.
//
// A block takes 64 tokens (one routing block: its masks are one 64-bit word per expert) and all of
// the experts (E <= 128 NB). Its 8 wavefronts split them as 2 token halves x 4 expert groups: each
// owns 32 tokens x 32 NB experts, NB blocks of v_mfma_f32_32x32x16_bf16 with fp32 accumulation over
// H in 64-deep K-tiles, which reach LDS by direct-to-LDS loads through a ring of S stages (the x rows
// stream from HBM once; W_r, 0.5 MB at E = 128, H = 2048, stays in L2). A K-tile carries little
// arithmetic (4 NB MFMAs per wave), so its fragment reads are issued a step ahead and two waves share
// each SIMD; with 4 waves of 64 tokens, each step waiting for its own reads, the kernel took 41 us at
// the 30B-A3B shape (1.9 TB/s), and a deeper ring alone did not change that.
#include "engine.h"
#include "moe_internal.h"
#include "route_device.h"

namespace moe {
namespace {

using namespace eng;

constexpr int RT = kRouteTokens;   // tokens per block
constexpr int RK = 64;             // contraction elements per K-tile: 128-byte rows

// 16-byte chunk c of row r of a staged K-tile: slot c ^ ((r >> 1) & 7), so that a ds_read_b128 of 16
// rows at one chunk is free of bank conflicts
__device__ __forceinline__ const char* kt_at(const char* tile, int r, int c) {
  return tile + r * 128 + ((c ^ ((r >> 1) & 7)) << 4);
}

// wait until at most n K-tiles of NL loads each are in flight (n <= N, a run-time value)
template <int NL, int N>
__device__ __forceinline__ void wait_ktiles(int n) {
  if constexpr (N == 0) {
    wait_vm<0>();
  } else {
    if (n >= N) wait_vm<N * NL>();
    else wait_ktiles<NL, N - 1>(n);
  }
}

template <int NB, int S>
__global__ __launch_bounds__(512, 1) void k_router_topk_bf16(RouteParams rp, const bf16* __restrict__ x,
                                                             const bf16* __restrict__ wr, float* __restrict__ lg_out,
                                                             int H) {
  constexpr int NE = 128 * NB;                  // expert rows per K-tile (W_r rows past E are clamped)
  constexpr int XB = RT * 128, STB = XB + NE * 128;
  constexpr int LDL = NE + 4;                   // staged logits row stride (floats): 4 banks mod 64
  constexpr int NL = 1 + 2 * NB;                // direct-to-LDS loads per lane per K-tile
  static_assert(RT * LDL * 4 <= S * STB, "the logits fit the ring");
  static_assert(S * STB + kMaxExperts * 8 <= 160 * 1024, "LDS");
  __shared__ __attribute__((aligned(1024))) char smem[S * STB];
  __shared__ unsigned long long mask[kMaxExperts];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, th = w >> 2, eg = w & 3;
  const int64_t t0 = (int64_t)blockIdx.x * RT;
  const int E = rp.E;
  for (int e = tid; e < rp.El; e += 512) mask[e] = 0ull;
  // This lane's row segments: x row 8w + lane/8 and W_r rows 16 NB w + 8i + lane/8 (i < 2 NB), chunk
  // (lane & 7) ^ swizzle; one wave instruction moves 8 whole 128-byte rows.
  const char* xp;
  const char* wp[2 * NB];
  {
    const int r = 8 * w + (lane >> 3);
    const int64_t tok = min(t0 + r, rp.T - 1);   // rows past T feed discarded outputs
    xp = reinterpret_cast<const char*>(x + tok * H) + 16 * ((lane & 7) ^ ((r >> 1) & 7));
  }
#pragma unroll
  for (int i = 0; i < 2 * NB; ++i) {
    const int r = 16 * NB * w + 8 * i + (lane >> 3);
    const int e = min(r, E - 1);                 // rows past E feed discarded outputs
    wp[i] = reinterpret_cast<const char*>(wr + (size_t)e * H) + 16 * ((lane & 7) ^ ((r >> 1) & 7));
  }
  auto issue = [&](int kt, char* st) {
    gl2lds(xp + (size_t)kt * 128, st + w * 1024);
#pragma unroll
    for (int i = 0; i < 2 * NB; ++i) gl2lds(wp[i] + (size_t)kt * 128, st + XB + (2 * NB * w + i) * 1024);
  };
  f32x16 acc[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j)
#pragma unroll
    for (int q = 0; q < 16; ++q) acc[j][q] = 0.f;
  const int arow = 32 * th + (lane & 31), brow = 32 * NB * eg + (lane & 31);
  auto frags = [&](const char* st, int ks, bf16x8& fa, bf16x8 (&fb)[NB]) {
    fa = *reinterpret_cast<const bf16x8*>(kt_at(st, arow, 2 * ks + (lane >> 5)));
#pragma unroll
    for (int j = 0; j < NB; ++j)
      fb[j] = *reinterpret_cast<const bf16x8*>(kt_at(st + XB, brow + 32 * j, 2 * ks + (lane >> 5)));
  };
  const int nk = H / RK;
#pragma unroll
  for (int q = 0; q < S; ++q)
    if (q < nk) issue(q, smem + q * STB);
  for (int kt = 0; kt < nk; ++kt) {
    wait_ktiles<NL, S - 1>(min(S - 1, nk - 1 - kt));   // K-tile kt has landed; the later ones may not
    block_sync();
    const char* st = smem + (kt % S) * STB;
    bf16x8 fa0, fb0[NB], fa1, fb1[NB];
    frags(st, 0, fa0, fb0);
#pragma unroll
    for (int ks = 0; ks < 4; ks += 2) {
      frags(st, ks + 1, fa1, fb1);   // the next step's fragments while this step multiplies
#pragma unroll
      for (int j = 0; j < NB; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb0[j], fa0, acc[j], 0, 0, 0);
      if (ks + 2 < 4) frags(st, ks + 2, fa0, fb0);
#pragma unroll
      for (int j = 0; j < NB; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb1[j], fa1, acc[j], 0, 0, 0);
    }
    block_sync();   // every wave is done with the stage
    if (kt + S < nk) issue(kt + S, smem + (kt % S) * STB);
  }
  // logits to LDS: accumulator element 4a + b of block j is token 32 th + (lane & 31), expert
  // 32 NB eg + 32 j + 8a + 4(lane >> 5) + b
  float* lg = reinterpret_cast<float*>(smem);
#pragma unroll
  for (int j = 0; j < NB; ++j)
#pragma unroll
    for (int a = 0; a < 4; ++a)
      *reinterpret_cast<float4*>(lg + arow * LDL + 32 * NB * eg + 32 * j + acc_n(a, lane)) =
          make_float4(acc[j][4 * a], acc[j][4 * a + 1], acc[j][4 * a + 2], acc[j][4 * a + 3]);
  __syncthreads();
  // the caller's logits [T, E]: the block's rows are contiguous
  const int nrow = (int)min((int64_t)RT, rp.T - t0);
  for (int q = tid; q < nrow * E; q += 512) {
    const int r = q / E, c = q - r * E;
    lg_out[t0 * E + q] = lg[r * LDL + c];
  }
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
  if (p.E <= 128) k_router_topk_bf16<1, 6><<<p.nblk, 512, 0, s>>>(p, xb, wb, logits, H);
  else k_router_topk_bf16<2, 3><<<p.nblk, 512, 0, s>>>(p, xb, wb, logits, H);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  prof_mark_end(s);
  return launch_route_tail(p, s);
}

}  // namespace moe
