// Routing: top-k expert selection, renormalised softmax weights, per-expert counts and offsets,
// the stable expert-major permutation of (token, slot) pairs, and the M-tile table of the
// grouped GEMMs. Dispatching tokens to experts is the first step of the fused layer ("A Magia da
// Fusão" on "IA: MoE Kernel 3x Mais Rápido Chegou!"), and the pages single out the sorting of
// tokens by expert as a cost ("kernel fuso per l'addestramento MoE" on "Prime Mega MoE: il kernel
// che accelera il training AI del 55%"). Experts are chosen by top-k over the fp32 logits, ties to
// the lower expert index. Weights are the softmax renormalised over the chosen k. Pairs are
// ordered by (local expert, t*k + j). The routing results are integers or come from a fixed
// sequence of fp32 operations, so runs are bitwise reproducible.
//
// Kernels (one stream, no host round trip):
//   k_route_topk     k <= 8: 64 tokens per block, 8 lanes per token; each lane sorts its eighth of
//                    the experts 8 at a time by sorting networks on 64-bit (logit, index) keys into
//                    a top-8 list, three shuffle steps merge the lists (route_device.h).
//   k_route_topk_wave  k > 8: one wavefront per token, k rounds of a wave-wide argmax.
//                    Both write, per block and local expert, a 64-bit mask of the tokens that chose it.
//   k_route_colscan  one block per local expert: exclusive scan of the per-block counts.
//   k_route_offsets  one block: expert offsets, M-tile tables and counts, and the offsets of the
//                    experts' padded segments (32 columns, 64 in the MX modes) in the
//                    pair-contiguous transposed copies.
//   k_route_scatter  one thread per pair: position = expert offset + earlier blocks' count +
//                    popcount of earlier tokens in the block's mask.
#include <math.h>

#include "moe_device.h"
#include "moe_internal.h"
#include "route_device.h"

namespace moe {

template <int NT>
__device__ __forceinline__ int block_incl_scan(int v, int* lds, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int n = __shfl_up(v, off);
    if (lane >= off) v += n;
  }
  if (lane == 63) lds[wave] = v;
  __syncthreads();
  int add = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) {
    const int x = lds[w];
    add += w < wave ? x : 0;
    tot += x;
  }
  __syncthreads();
  total = tot;
  return v + add;
}

// k <= 8: 64 tokens per block, LPT lanes per token (route_token). LPT = 8 took 20 us against 23 us
// with 4 at T = 16384, E = 128 (one candidate inserted at a time; the sorting networks then took it
// to 14.5 us); LPT = 16 sent the compiler into a build of more than 15 minutes.
template <int KMAX, int LPT>
__global__ __launch_bounds__(64 * LPT) void k_route_topk(RouteParams p) {
  constexpr int NT = 64 * LPT;
  __shared__ unsigned long long mask[kMaxExperts];
  const int tid = threadIdx.x, tl = tid / LPT, q = tid % LPT;
  for (int e = tid; e < p.El; e += NT) mask[e] = 0ull;
  __syncthreads();
  const int64_t t = (int64_t)blockIdx.x * kRouteTokens + tl;
  if (t < p.T) {
    const float* row = p.logits + t * p.E;
    route_token<KMAX, LPT>(p, t, tl, q, [&](int e) { return row[e]; }, mask);
  }
  __syncthreads();
  for (int e = tid; e < p.El; e += NT) {
    const size_t qq = (size_t)blockIdx.x * p.El + e;
    p.blk_mask[qq] = mask[e];
    p.blk_count[qq] = __popcll(mask[e]);
  }
}

// k > 8: one wavefront per token, k rounds of a wave-wide (value desc, index asc) argmax.
template <int PER_LANE>
__global__ __launch_bounds__(256) void k_route_topk_wave(RouteParams p) {
  __shared__ unsigned long long mask[kMaxExperts];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  for (int e = tid; e < p.El; e += 256) mask[e] = 0ull;
  __syncthreads();
  const int64_t t_base = (int64_t)blockIdx.x * kRouteTokens;
  for (int tl = wave; tl < kRouteTokens; tl += 4) {
    const int64_t t = t_base + tl;
    if (t >= p.T) break;
    const float* row = p.logits + t * p.E;
    float v[PER_LANE];
#pragma unroll
    for (int i = 0; i < PER_LANE; ++i) {
      const int e = lane + 64 * i;
      v[i] = e < p.E ? row[e] : -INFINITY;
    }
    unsigned taken = 0;
    float top = 0.f, my_v = 0.f;
    int my_e = -1;
    for (int j = 0; j < p.k; ++j) {
      float bv = -INFINITY;
      int be = 0x7fffffff;
#pragma unroll
      for (int i = 0; i < PER_LANE; ++i) {
        const int e = lane + 64 * i;
        if (e < p.E && !((taken >> i) & 1u) && better(v[i], e, bv, be)) {
          bv = v[i];
          be = e;
        }
      }
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) {
        const float ov = __shfl_xor(bv, off);
        const int oe = __shfl_xor(be, off);
        if (better(ov, oe, bv, be)) {
          bv = ov;
          be = oe;
        }
      }
      if ((be & 63) == lane) taken |= 1u << (be >> 6);
      if (lane == j) {
        my_v = bv;
        my_e = be;
      }
      if (j == 0) top = bv;
    }
    const float z = lane < p.k ? expf(my_v - top) : 0.f;
    float s = z;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off);
    s = __shfl(s, 0);
    if (lane < p.k) {
      p.idx[t * p.k + lane] = my_e;
      p.weight[t * p.k + lane] = z / s;
      const int el = my_e - p.e0;
      if (el >= 0 && el < p.El) atomicOr(&mask[el], 1ull << tl);
    }
  }
  __syncthreads();
  for (int e = tid; e < p.El; e += 256) {
    const size_t q = (size_t)blockIdx.x * p.El + e;
    p.blk_mask[q] = mask[e];
    p.blk_count[q] = __popcll(mask[e]);
  }
}

__global__ __launch_bounds__(256) void k_route_colscan(RouteParams p) {
  __shared__ int lds[4];
  const int e = blockIdx.x, tid = threadIdx.x;
  int carry = 0;
  for (int b0 = 0; b0 < p.nblk; b0 += 256) {
    const int b = b0 + tid;
    const int c = b < p.nblk ? p.blk_count[(size_t)b * p.El + e] : 0;
    int tot;
    const int incl = block_incl_scan<256>(c, lds, tot);
    if (b < p.nblk) p.blk_prefix[(size_t)b * p.El + e] = carry + incl - c;
    carry += tot;
  }
  if (tid == 0) p.counts[e] = carry;
}

__global__ __launch_bounds__(512) void k_route_offsets(RouteParams p) {
  __shared__ int lds[8];
  const int e = threadIdx.x;
  const int c = e < p.El ? p.counts[e] : 0;
  const int nt = (c + kBM - 1) / kBM, nt2 = (c + kBM2 - 1) / kBM2;
  const int c32 = (c + p.qpad - 1) & ~(p.qpad - 1);
  int tot_c, tot_t, tot_t2, tot_q;
  const int inc_c = block_incl_scan<512>(c, lds, tot_c);
  const int inc_t = block_incl_scan<512>(nt, lds, tot_t);
  const int inc_t2 = block_incl_scan<512>(nt2, lds, tot_t2);
  const int inc_q = block_incl_scan<512>(c32, lds, tot_q);
  if (e < p.El) {
    const int off = inc_c - c, t0 = inc_t - nt, t2 = inc_t2 - nt2;
    p.offsets[e] = off;
    p.qoff[e] = inc_q - c32;
    for (int i = 0; i < nt; ++i) p.mtile[t0 + i] = make_int2(e, off + i * kBM);
    for (int i = 0; i < nt2; ++i) p.mtile2[t2 + i] = make_int2(e, off + i * kBM2);
  }
  if (e == 0) {
    p.offsets[p.El] = tot_c;
    p.qoff[p.El] = tot_q;
    *p.num_mtiles = tot_t;
    *p.num_mtiles2 = tot_t2;
  }
  if (e < kZeroBytes / 16) p.zeros[e] = make_uint4(0u, 0u, 0u, 0u);
  if (e < kSchedSlots * kSchedInts) p.sched[e] = 0;
}

__global__ __launch_bounds__(256) void k_route_scatter(RouteParams p) {
  const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (q >= p.T * p.k) return;
  const int64_t t = q / p.k;
  const int el = p.idx[q] - p.e0;
  if (el < 0 || el >= p.El) {
    p.pair_pos[q] = -1;
    return;
  }
  const int b = (int)(t / kRouteTokens), tl = (int)(t % kRouteTokens);
  const size_t cell = (size_t)b * p.El + el;
  const unsigned long long before = p.blk_mask[cell] & ((1ull << tl) - 1ull);
  const int pos = p.offsets[el] + p.blk_prefix[cell] + __popcll(before);
  p.perm[pos] = (int)q;
  p.ptok[pos] = (int)t;
  p.pair_pos[q] = pos;
}

hipError_t launch_route(const RouteParams& p, hipStream_t s) {
  hipError_t err;
  prof_mark_begin("route_topk", s);
  const int per_lane = (p.E + 63) / 64;
  if (p.k <= 8) k_route_topk<8, 8><<<p.nblk, 64 * 8, 0, s>>>(p);
  else if (per_lane <= 1) k_route_topk_wave<1><<<p.nblk, 256, 0, s>>>(p);
  else if (per_lane <= 2) k_route_topk_wave<2><<<p.nblk, 256, 0, s>>>(p);
  else if (per_lane <= 4) k_route_topk_wave<4><<<p.nblk, 256, 0, s>>>(p);
  else k_route_topk_wave<8><<<p.nblk, 256, 0, s>>>(p);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  prof_mark_end(s);
  return launch_route_tail(p, s);
}

// after the top-k: per-expert scans, offsets and M-tile tables, and the permutation
hipError_t launch_route_tail(const RouteParams& p, hipStream_t s) {
  hipError_t err;
  prof_mark_begin("route_colscan", s);
  k_route_colscan<<<p.El, 256, 0, s>>>(p);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  prof_mark_end(s);
  prof_mark_begin("route_offsets", s);
  k_route_offsets<<<1, 512, 0, s>>>(p);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  prof_mark_end(s);
  const int64_t pairs = p.T * p.k;
  prof_mark_begin("route_scatter", s);
  k_route_scatter<<<(unsigned)((pairs + 255) / 256), 256, 0, s>>>(p);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  prof_mark_end(s);
  return hipSuccess;
}

}  // namespace moe
