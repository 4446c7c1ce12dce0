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

// Insert candidate (cv, ce) into the list t[0..KMAX) kept sorted by better(); the loser of each
// compare-exchange moves on. Branchless.
template <int KMAX>
__device__ __forceinline__ void topk_insert(float (&tv)[KMAX], int (&ti)[KMAX], float cv, int ce) {
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    const bool b = better(cv, ce, tv[j], ti[j]);
    const float nv = b ? cv : tv[j];
    const int ni = b ? ce : ti[j];
    cv = b ? tv[j] : cv;
    ce = b ? ti[j] : ce;
    tv[j] = nv;
    ti[j] = ni;
  }
}

// Top-k of token t (k <= KMAX) by its LPT lanes: lane q keeps the best KMAX of experts q, q+LPT,
// q+2 LPT, ... (logit e from get(e)); log2(LPT) butterfly steps merge the lists, after which every lane
// of the token holds its top k. Writes the token's expert indices and renormalised softmax weights
// (summed in slot order) and sets its bit (tl) in the block's per-local-expert masks.
template <int KMAX, int LPT, class Get>
__device__ __forceinline__ void route_token(const RouteParams& p, int64_t t, int tl, int q, Get get,
                                            unsigned long long* mask) {
  float tv[KMAX];
  int ti[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    tv[j] = -INFINITY;
    ti[j] = 0x7fffffff;
  }
  // 8 of the lane's logits are read at a time, then inserted: the loads of a batch are in flight
  // together (one at a time, each insertion waited for its own load)
  for (int e0 = q; e0 < p.E; e0 += 8 * LPT) {
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = e0 + i * LPT < p.E ? get(e0 + i * LPT) : -INFINITY;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (e0 + i * LPT < p.E) topk_insert<KMAX>(tv, ti, v[i], e0 + i * LPT);
  }
  // merge with the partner lane's list: the better of tv[j] and the partner's [KMAX-1-j]
  // leaves the top KMAX of both lists as a bitonic sequence, which three half-cleaner stages sort
#pragma unroll
  for (int step = 1; step < LPT; step <<= 1) {
    float ov[KMAX];
    int oi[KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      ov[j] = __shfl_xor(tv[j], step);
      oi[j] = __shfl_xor(ti[j], step);
    }
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      const bool b = better(tv[j], ti[j], ov[KMAX - 1 - j], oi[KMAX - 1 - j]);
      tv[j] = b ? tv[j] : ov[KMAX - 1 - j];
      ti[j] = b ? ti[j] : oi[KMAX - 1 - j];
    }
#pragma unroll
    for (int d = KMAX / 2; d >= 1; d >>= 1)
#pragma unroll
      for (int j = 0; j < KMAX; ++j)
        if ((j & d) == 0) {
          const bool b = better(tv[j], ti[j], tv[j + d], ti[j + d]);
          const float v0 = b ? tv[j] : tv[j + d], v1 = b ? tv[j + d] : tv[j];
          const int i0 = b ? ti[j] : ti[j + d], i1 = b ? ti[j + d] : ti[j];
          tv[j] = v0;
          tv[j + d] = v1;
          ti[j] = i0;
          ti[j + d] = i1;
        }
  }
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
