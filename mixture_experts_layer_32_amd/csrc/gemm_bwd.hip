// Backward of the fused MoE layer: the pass Prime added to DeepSeek's forward-only kernel
// ("Afinal, o que é esse Prime Mega MoE?" on "IA: MoE Kernel 3x Mais Rápido Chegou!"; "Qué se ha
// publicado" on the ai-daily-news.org page).
//
// The forward saved, per routed pair r (expert-sorted order), a = x W_gate^T, b = x W_up^T and
// hw = w_r silu(a) b. With u = W_down[e]^T dY_t:
//   k_bwd_dh         row-tiled: u = gather(dY) W_down[e] (contraction over H). The epilogue
//                    recomputes h = silu(a) b and writes
//                      g partials   <u, h> per 64-column slice
//                      da           w u b silu'(a)
//                      db           w u silu(a)
//   k_wgrad_down     per expert: dW_down[e] = sum_r dY_t hw_r^T. Contraction over the expert's
//                    rows; both operands are contiguous along M or N and are transposed on
//                    their way into LDS.
//   k_wgrad_gateup   per expert: [dW_gate; dW_up][e] = sum_r [da; db]_r x_t^T.
//   k_dgrad_x        row-tiled: dX_r = [da db]_r [W_gate[e]; W_up[e]] (contraction over 2F).
//   k_combine_bwd    dx_t = sum over local slots of dX; dlogits through the renormalised
//                    softmax, with g_tj = sum of the partials = <dY_t, o_tj>.
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

// contraction row k of W_down[e] restricted to columns [n0, n0+128): contiguous along F
template <class T>
struct WdRows {
  const T* base;  // wd + e*H*F + n0
  int F;
  __device__ __forceinline__ const char* row(int k) const {
    return reinterpret_cast<const char*>(base + (size_t)k * F);
  }
};

// contraction row k of [W_gate[e]; W_up[e]] (2F rows of length H) restricted to [n0, n0+128)
template <class T>
struct GateUpRows {
  const T* g;  // wg + e*F*H + n0
  const T* u;  // wu + e*F*H + n0
  int F, H;
  __device__ __forceinline__ const char* row(int k) const {
    return reinterpret_cast<const char*>(k < F ? g + (size_t)k * H : u + (size_t)(k - F) * H);
  }
};

// contraction row k = expert-local pair index: token row of a [T, ld] tensor, via perm
template <class T>
struct GatherRows {
  const T* base;  // tensor + c0
  const int* ptok;
  int seg0, seg_end, ld;
  __device__ __forceinline__ const char* row(int k) const {
    const int r = seg0 + k;
    return r < seg_end ? reinterpret_cast<const char*>(base + (size_t)ptok[r] * ld) : nullptr;
  }
};

// contraction row k = expert-local pair index: row seg0+k of a pair-indexed [rows, ld] tensor
template <class T>
struct PairRows {
  const T* base;  // tensor + c0
  int seg0, seg_end, ld;
  __device__ __forceinline__ const char* row(int k) const {
    const int r = seg0 + k;
    return r < seg_end ? reinterpret_cast<const char*>(base + (size_t)r * ld) : nullptr;
  }
};

template <class T>
__global__ __launch_bounds__(kThreads, 2) void k_bwd_dh(BwdParams p) {
  __shared__ __attribute__((aligned(16))) char smem[kSmemBytes];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1;
  const T* __restrict__ dy = static_cast<const T*>(p.dy);
  const T* __restrict__ wd = static_cast<const T*>(p.wd);
  const T* __restrict__ ab = static_cast<const T*>(p.ab);
  T* __restrict__ dab = static_cast<T*>(p.dab);
  const int H = p.H, F = p.F;
  const int ntn = F / 128;
  const int total = *p.num_mtiles * ntn;
  const int nk = H / Elem<T>::BK;
  const XcdRange xr = xcd_range(total);
  const int brow[4] = {wn * 64, wn * 64 + 16, wn * 64 + 32, wn * 64 + 48};
  for (int tile = xr.first; tile < xr.end; tile += xr.stride) {
    const int mt = tile / ntn, nt = tile - mt * ntn;
    const int2 me = p.mtile[mt];
    const int e = me.x, r0 = me.y;
    const int seg_end = p.offsets[e + 1];
    KLoader<128> la;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = r0 + (tid >> 3) + 32 * i;
      la.p[i] = r < seg_end ? reinterpret_cast<const char*>(dy + (size_t)p.ptok[r] * H) + (tid & 7) * 16
                            : nullptr;
    }
    MNLoader<T, 128, WdRows<T>> lb;
    lb.src = WdRows<T>{wd + (size_t)e * H * F + nt * 128, F};
    lb.init(tid);
    f32x4 acc[4][4];
    mainloop<T>(acc, smem, la, lb, nk, wm * 64, brow);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int r = r0 + wm * 64 + i * 16 + 4 * (lane >> 4) + q;
        const bool valid = r < seg_end;
        const float w = valid ? p.weight[p.perm[r]] : 0.f;
        float gsum = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int f = nt * 128 + wn * 64 + j * 16 + (lane & 15);
          if (valid) {
            const float av = (float)ab[(size_t)r * 2 * F + f];
            const float bv = (float)ab[(size_t)r * 2 * F + F + f];
            const float sg = sigmoidf_(av);
            const float si = av * sg;
            const float u = acc[i][j][q];
            gsum += u * (si * bv);
            const float dh = w * u;
            dab[(size_t)r * 2 * F + f] = cvt_out<T>(dh * bv * sg * (1.0f + av * (1.0f - sg)));
            dab[(size_t)r * 2 * F + F + f] = cvt_out<T>(dh * si);
          }
        }
        gsum += __shfl_xor(gsum, 1);
        gsum += __shfl_xor(gsum, 2);
        gsum += __shfl_xor(gsum, 4);
        gsum += __shfl_xor(gsum, 8);
        if (valid && (lane & 15) == 0) p.gpart[(size_t)(nt * 2 + wn) * p.rows + r] = gsum;
      }
    }
  }
}

template <class T>
__global__ __launch_bounds__(kThreads, 2) void k_dgrad_x(BwdParams p) {
  __shared__ __attribute__((aligned(16))) char smem[kSmemBytes];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1;
  const T* __restrict__ dab = static_cast<const T*>(p.dab);
  const T* __restrict__ wg = static_cast<const T*>(p.wg);
  const T* __restrict__ wu = static_cast<const T*>(p.wu);
  T* __restrict__ dxp = static_cast<T*>(p.dxp);
  const int H = p.H, F = p.F;
  const int ntn = H / 128;
  const int total = *p.num_mtiles * ntn;
  const int nk = 2 * F / Elem<T>::BK;
  const XcdRange xr = xcd_range(total);
  const int brow[4] = {wn * 64, wn * 64 + 16, wn * 64 + 32, wn * 64 + 48};
  for (int tile = xr.first; tile < xr.end; tile += xr.stride) {
    const int mt = tile / ntn, nt = tile - mt * ntn;
    const int2 me = p.mtile[mt];
    const int e = me.x, r0 = me.y;
    const int seg_end = p.offsets[e + 1];
    KLoader<128> la;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = r0 + (tid >> 3) + 32 * i;
      la.p[i] = r < seg_end ? reinterpret_cast<const char*>(dab + (size_t)r * 2 * F) + (tid & 7) * 16 : nullptr;
    }
    MNLoader<T, 128, GateUpRows<T>> lb;
    lb.src = GateUpRows<T>{wg + (size_t)e * F * H + nt * 128, wu + (size_t)e * F * H + nt * 128, F, H};
    lb.init(tid);
    f32x4 acc[4][4];
    mainloop<T>(acc, smem, la, lb, nk, wm * 64, brow);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int r = r0 + wm * 64 + i * 16 + 4 * (lane >> 4) + q;
        if (r >= seg_end) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int n = nt * 128 + wn * 64 + j * 16 + (lane & 15);
          dxp[(size_t)r * H + n] = cvt_out<T>(acc[i][j][q]);
        }
      }
    }
  }
}

// dW_down[e] (H x F) = sum over the expert's pairs r of dY_{t_r} hw_r^T
template <class T>
__global__ __launch_bounds__(kThreads, 2) void k_wgrad_down(BwdParams p) {
  __shared__ __attribute__((aligned(16))) char smem[kSmemBytes];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1;
  const int H = p.H, F = p.F;
  const int ntn = F / 128, tpe = (H / 128) * ntn;
  const int lid = xcd_logical_block(gridDim.x);
  const int e = lid / tpe, t = lid - e * tpe;
  const int mt = t / ntn, nt = t - mt * ntn;
  const int seg0 = p.offsets[e], seg_end = p.offsets[e + 1];
  const int nk = (seg_end - seg0 + Elem<T>::BK - 1) / Elem<T>::BK;
  MNLoader<T, 128, GatherRows<T>> la;
  la.src = GatherRows<T>{static_cast<const T*>(p.dy) + mt * 128, p.ptok, seg0, seg_end, H};
  la.init(tid);
  MNLoader<T, 128, PairRows<T>> lb;
  lb.src = PairRows<T>{static_cast<const T*>(p.hw) + nt * 128, seg0, seg_end, F};
  lb.init(tid);
  const int brow[4] = {wn * 64, wn * 64 + 16, wn * 64 + 32, wn * 64 + 48};
  f32x4 acc[4][4];
  mainloop<T>(acc, smem, la, lb, nk, wm * 64, brow);
  T* __restrict__ out = static_cast<T*>(p.dwd) + (size_t)e * H * F;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int m = mt * 128 + wm * 64 + i * 16 + 4 * (lane >> 4) + q;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int n = nt * 128 + wn * 64 + j * 16 + (lane & 15);
        out[(size_t)m * F + n] = cvt_out<T>(acc[i][j][q]);
      }
    }
}

// [dW_gate; dW_up][e] (2F x H) = sum over the expert's pairs r of [da; db]_r x_{t_r}^T
template <class T>
__global__ __launch_bounds__(kThreads, 2) void k_wgrad_gateup(BwdParams p) {
  __shared__ __attribute__((aligned(16))) char smem[kSmemBytes];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1;
  const int H = p.H, F = p.F;
  const int ntn = H / 128, tpe = (2 * F / 128) * ntn;
  const int lid = xcd_logical_block(gridDim.x);
  const int e = lid / tpe, t = lid - e * tpe;
  const int mt = t / ntn, nt = t - mt * ntn;
  const int seg0 = p.offsets[e], seg_end = p.offsets[e + 1];
  const int nk = (seg_end - seg0 + Elem<T>::BK - 1) / Elem<T>::BK;
  MNLoader<T, 128, PairRows<T>> la;
  la.src = PairRows<T>{static_cast<const T*>(p.dab) + mt * 128, seg0, seg_end, 2 * F};
  la.init(tid);
  MNLoader<T, 128, GatherRows<T>> lb;
  lb.src = GatherRows<T>{static_cast<const T*>(p.x) + nt * 128, p.ptok, seg0, seg_end, H};
  lb.init(tid);
  const int brow[4] = {wn * 64, wn * 64 + 16, wn * 64 + 32, wn * 64 + 48};
  f32x4 acc[4][4];
  mainloop<T>(acc, smem, la, lb, nk, wm * 64, brow);
  const bool gate = mt * 128 < F;
  T* __restrict__ out = static_cast<T*>(gate ? p.dwg : p.dwu) + (size_t)e * F * H;
  const int m0 = gate ? mt * 128 : mt * 128 - F;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int m = m0 + wm * 64 + i * 16 + 4 * (lane >> 4) + q;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int n = nt * 128 + wn * 64 + j * 16 + (lane & 15);
        out[(size_t)m * H + n] = cvt_out<T>(acc[i][j][q]);
      }
    }
}

// One wavefront per part of a row (128 chunks of 16 bytes) of tpw consecutive tokens (combine_tpw), 4
// wavefronts per block, as in the forward combine; part 0 also writes those tokens' dlogits. Lane
// q < (tokens) k holds slot q % k of token q / k: its pair position, weight, expert and g = the sum of
// its partials. Slot values reach every lane through readlane, so a token's k source rows are
// addressed from scalar registers.
template <class T>
__global__ __launch_bounds__(256) void k_combine_bwd(BwdParams p, int tpw) {
  constexpr int VEC = Elem<T>::VEC;
  const int lane = threadIdx.x & 63;
  const int k = p.k, H = p.H;
  const int nch = H / VEC, nparts = (nch + 127) / 128;
  const int64_t u = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t tg = u / nparts;
  const int part = (int)(u - tg * nparts);
  const int64_t t0 = tg * tpw;
  if (t0 >= p.T) return;   // the whole wave leaves
  const int nt = (int)min((int64_t)tpw, p.T - t0);
  const bool mine = lane < nt * k;
  const int pp = mine ? p.pair_pos[t0 * k + lane] : -1;
  // dx_t = sum over the local slots of dX' rows, fp32 in slot order
  for (int tt = 0; tt < nt; ++tt)
    combine_row_part<T, VEC>(static_cast<const T*>(p.dxp), pp, tt * k, k, H, nch, part, nparts, lane,
                             static_cast<T*>(p.dx) + (t0 + tt) * H);
  // dlogits of the tokens, by part 0, after its share of dx (the other parts skip the partials)
  if (part != 0) return;
  int ex = -1;
  float w = 0.f, g = 0.f;
  if (mine) {
    w = p.weight[t0 * k + lane];
    ex = p.idx[t0 * k + lane];
    if (pp >= 0)
      for (int q = 0; q < p.np; ++q) g += p.gpart[(size_t)q * p.rows + pp];
  }
  const float wg = w * g;
  for (int tt = 0; tt < nt; ++tt) {
    // gbar = sum_j w_j g_j over the token's slots, in slot order
    float gbar = 0.f;
    for (int j = 0; j < k; ++j)
      gbar += __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wg), tt * k + j));
    const float val = w * (g - gbar);   // dlogits of slot q's expert, meaningful in the token's lanes
    float* row = p.dlogits + (t0 + tt) * p.E;
    // uniform over the wave, so that every lane is active at the readlane (the token's lanes can lie
    // past E, where a loop over e < E would leave val uncomputed)
    for (int eb = 0; eb < p.E; eb += 64) {
      const int e = eb + lane;
      float v = 0.f;
      for (int j = 0; j < k; ++j)
        if (__builtin_amdgcn_readlane(ex, tt * k + j) == e)
          v = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, val), tt * k + j));
      if (e < p.E) row[e] = v;
    }
  }
}

template <class T>
hipError_t launch_backward(const BwdParams& p, int grid, hipStream_t s) {
  hipError_t err;
  prof_mark_begin("gemm_bwd_dh_dswiglu", s);
  k_bwd_dh<T><<<grid, kThreads, 0, s>>>(p);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  prof_mark_end(s);

  const int nb_wd = p.El * (p.H / 128) * (p.F / 128);
  prof_mark_begin("gemm_wgrad_down", s);
  k_wgrad_down<T><<<nb_wd, kThreads, 0, s>>>(p);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  prof_mark_end(s);

  const int nb_wgu = p.El * (2 * p.F / 128) * (p.H / 128);
  prof_mark_begin("gemm_wgrad_gateup", s);
  k_wgrad_gateup<T><<<nb_wgu, kThreads, 0, s>>>(p);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  prof_mark_end(s);

  prof_mark_begin("gemm_dgrad_x", s);
  k_dgrad_x<T><<<grid, kThreads, 0, s>>>(p);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  prof_mark_end(s);
  return hipSuccess;
}

template <class T>
hipError_t launch_combine_bwd(const BwdParams& p, hipStream_t s) {
  prof_mark_begin("combine_bwd", s);
  const int64_t nparts = (p.H / Elem<T>::VEC + 127) / 128, tpw = combine_tpw(p.k, p.El, p.E);
  const int64_t waves = (p.T + tpw - 1) / tpw * nparts;
  k_combine_bwd<T><<<(unsigned)((waves + 3) / 4), 256, 0, s>>>(p, (int)tpw);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  prof_mark_end(s);
  return hipSuccess;
}

template hipError_t launch_backward<float>(const BwdParams&, int, hipStream_t);
template hipError_t launch_combine_bwd<float>(const BwdParams&, hipStream_t);
template hipError_t launch_combine_bwd<bf16>(const BwdParams&, hipStream_t);

}  // namespace moe
