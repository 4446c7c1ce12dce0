// Per-token top-k selection of the routing, shared by the routing kernels (logits from memory) and the
// router projection fused with the routing (logits from LDS). Experts are chosen by top-k over the
// fp32 logits, ties to the lower expert index ("Os Números que Impressionam" on "IA: MoE Kernel 3x
// Mais Rápido Chegou!": top-8 of 128 experts); the weights are the softmax renormalised over the
// chosen k.
#pragma once
#include <math.h>

#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

__device__ __forceinline__ bool better(float av, int ae, float bv, int be) {
  return av > bv || (av == bv && ae < be);
}

// Order-preserving 64-bit key of (logit v, expert e): a larger key is a better candidate (larger logit,
// then lower index). The high word maps the fp32 bits monotonically to unsigned order, with -0 taken
// as +0 so that the two zeros tie as equal logits do; the low word is ~e. Finite logits only.
__device__ __forceinline__ unsigned long long topk_key(float v, int e) {
  unsigned u = __float_as_uint(v);
  u = u == 0x80000000u ? 0u : u;
  const unsigned o = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((unsigned long long)o << 32) | (unsigned)~e;
}
__device__ __forceinline__ float key_value(unsigned long long k) {
  const unsigned o = (unsigned)(k >> 32);
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7fffffffu) : ~o);
}
__device__ __forceinline__ int key_expert(unsigned long long k) { return (int)~(unsigned)k; }

// compare-exchange into descending order
__device__ __forceinline__ void key_ce(unsigned long long& a, unsigned long long& b) {
  const bool s = b > a;
  const unsigned long long hi = s ? b : a, lo = s ? a : b;
  a = hi;
  b = lo;
}
// sorts 8 keys into descending order: Knuth's 19-comparator network for 8 inputs, in 6 parallel rounds
__device__ __forceinline__ void key_sort8(unsigned long long (&k)[8]) {
  key_ce(k[0], k[2]); key_ce(k[1], k[3]); key_ce(k[4], k[6]); key_ce(k[5], k[7]);
  key_ce(k[0], k[4]); key_ce(k[1], k[5]); key_ce(k[2], k[6]); key_ce(k[3], k[7]);
  key_ce(k[0], k[1]); key_ce(k[2], k[3]); key_ce(k[4], k[5]); key_ce(k[6], k[7]);
  key_ce(k[2], k[4]); key_ce(k[3], k[5]);
  key_ce(k[1], k[4]); key_ce(k[3], k[6]);
  key_ce(k[1], k[2]); key_ce(k[3], k[4]); key_ce(k[5], k[6]);
}
// t (descending) becomes the best 8 of t and c (both descending): the larger of t[j] and c[7-j] leaves
// the best 8 as a bitonic sequence, which three half-cleaner rounds sort
__device__ __forceinline__ void key_merge8(unsigned long long (&t)[8], const unsigned long long (&c)[8]) {
#pragma unroll
  for (int j = 0; j < 8; ++j) t[j] = t[j] > c[7 - j] ? t[j] : c[7 - j];
#pragma unroll
  for (int d = 4; d >= 1; d >>= 1)
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if ((j & d) == 0) key_ce(t[j], t[j + d]);
}

// t becomes the merge of t and the list of the lane that DPP control CTRL selects (a butterfly step:
// the merge is symmetric, so both lanes end with the same list)
template <int CTRL>
__device__ __forceinline__ void merge_partner(unsigned long long (&t)[8]) {
  unsigned long long o[8];
#pragma unroll
  for (int j = 0; j < 8; ++j)
    o[j] = ((unsigned long long)dpp_mov<CTRL>((unsigned)(t[j] >> 32)) << 32) | dpp_mov<CTRL>((unsigned)t[j]);
  key_merge8(t, o);
}

// Best 8 of experts 0..E-1 (logit e from get(e)) by LPT lanes of a token, lane q taking experts q,
// q + LPT, ...: each lane sorts its candidates 8 at a time and merges them into its list, then log2(LPT)
// butterfly steps merge the lanes' lists (DPP moves: partners xor 1, xor 2, then the mirrored lane of
// the 8, which after the quad steps holds the same list as the xor-4 one), after which every lane of
// the token holds the token's best 8 (slots past E hold key 0 and come last). The token's lanes must
// all be active.
template <int LPT, class Get>
__device__ __forceinline__ void select_top8(int E, int q, Get get, float (&tv)[8], int (&ti)[8]) {
  unsigned long long t[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) t[j] = 0ull;
  for (int e0 = q; e0 < E; e0 += 8 * LPT) {
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = e0 + i * LPT < E ? get(e0 + i * LPT) : 0.f;
    unsigned long long c[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) c[i] = e0 + i * LPT < E ? topk_key(v[i], e0 + i * LPT) : 0ull;
    key_sort8(c);
    key_merge8(t, c);
  }
  static_assert(LPT == 1 || LPT == 2 || LPT == 4 || LPT == 8, "lanes per token");
  if constexpr (LPT > 1) merge_partner<kDppXor1>(t);
  if constexpr (LPT > 2) merge_partner<kDppXor2>(t);
  if constexpr (LPT > 4) merge_partner<kDppHalfMirror>(t);   // the quads' lists are merged by now
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    tv[j] = key_value(t[j]);
    ti[j] = key_expert(t[j]);
  }
}

// Top-k of token t (k <= KMAX = 8) by its LPT lanes (select_top8), after which every lane of the
// token holds its top k. Writes the token's expert indices and renormalised softmax weights
// (summed in slot order) and sets its bit (tl) in the block's per-local-expert masks.
template <int KMAX, int LPT, class Get>
__device__ __forceinline__ void route_token(const RouteParams& p, int64_t t, int tl, int q, Get get,
                                            unsigned long long* mask) {
  static_assert(KMAX == 8, "the selection keeps the best 8");
  float tv[KMAX];
  int ti[KMAX];
  select_top8<LPT>(p.E, q, get, tv, ti);
  // renormalised softmax over the chosen k, summed in slot order
  float z[KMAX], sum = 0.f;
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    z[j] = j < p.k ? expf(tv[j] - tv[0]) : 0.f;
    sum += z[j];
  }
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    if (j < p.k && (j & (LPT - 1)) == q) {
      p.idx[t * p.k + j] = ti[j];
      p.weight[t * p.k + j] = z[j] / sum;
      const int el = ti[j] - p.e0;
      if (el >= 0 && el < p.El) atomicOr(&mask[el], 1ull << tl);
    }
  }
}

}  // namespace moe
