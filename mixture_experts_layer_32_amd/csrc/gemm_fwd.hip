// Forward expert computation. "A Magia da Fusão" on "IA: MoE Kernel 3x Mais Rápido Chegou!" lists
// it: the experts' linear layers with SwiGLU between them, then the combine of the expert outputs.
// "Detalhes Técnicos Rápidos" on the same page requires gated SwiGLU experts without biases.
//
//   k_gateup   persistent grouped GEMM over (M-tile of an expert's rows, 64-column slice of F).
//              A = x rows gathered through the permutation, so the dispatched copy of x is never
//              stored. B = the matching 64 rows of W_gate[e] and 64 rows of W_up[e].
//              Epilogue: a, b (saved for the backward) and hw = w_r * silu(a) * b.
//   k_down     persistent grouped GEMM: o'[r] = hw[r] W_down[e]^T. The routing weight is
//              already in hw.
//   k_combine  y_t = sum over the token's local slots of o'[pair_pos]. Gather-sum, fp32
//              accumulation, one wavefront per token, 16-byte coalesced row reads.
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

template <class T>
__global__ __launch_bounds__(kThreads, 2) void k_gateup(FwdParams p) {
  __shared__ __attribute__((aligned(16))) char smem[kSmemBytes];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1;
  const T* __restrict__ x = static_cast<const T*>(p.x);
  const T* __restrict__ wg = static_cast<const T*>(p.wg);
  const T* __restrict__ wu = static_cast<const T*>(p.wu);
  T* __restrict__ ab = static_cast<T*>(p.ab);
  T* __restrict__ hw = static_cast<T*>(p.hw);
  const int H = p.H, F = p.F;
  const int ntn = F / 64;
  const int total = *p.num_mtiles * ntn;
  const int nk = H / Elem<T>::BK;
  const XcdRange xr = xcd_range(total);
  const int brow[4] = {wn * 32, wn * 32 + 16, 64 + wn * 32, 64 + wn * 32 + 16};
  for (int tile = xr.first; tile < xr.end; tile += xr.stride) {
    const int mt = tile / ntn, nt = tile - mt * ntn;
    const int2 me = p.mtile[mt];
    const int e = me.x, r0 = me.y;
    const int seg_end = p.offsets[e + 1];
    KLoader<128> la, lb;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = (tid >> 3) + 32 * i;
      const int r = r0 + row;
      la.p[i] = r < seg_end ? reinterpret_cast<const char*>(x + (size_t)p.ptok[r] * H) + (tid & 7) * 16
                            : nullptr;
      const T* wrow = row < 64 ? wg + ((size_t)e * F + nt * 64 + row) * H
                               : wu + ((size_t)e * F + nt * 64 + row - 64) * H;
      lb.p[i] = reinterpret_cast<const char*>(wrow) + (tid & 7) * 16;
    }
    f32x4 acc[4][4];
    mainloop<T>(acc, smem, la, lb, nk, wm * 64, brow);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int r = r0 + wm * 64 + i * 16 + 4 * (lane >> 4) + q;
        if (r >= seg_end) continue;
        const float w = p.weight[p.perm[r]];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int f = nt * 64 + wn * 32 + j * 16 + (lane & 15);
          const float av = acc[i][j][q], bv = acc[i][j + 2][q];
          const float h = av * sigmoidf_(av) * bv;
          ab[(size_t)r * 2 * F + f] = cvt_out<T>(av);
          ab[(size_t)r * 2 * F + F + f] = cvt_out<T>(bv);
          hw[(size_t)r * F + f] = cvt_out<T>(w * h);
        }
      }
    }
  }
}

template <class T>
__global__ __launch_bounds__(kThreads, 2) void k_down(FwdParams p) {
  __shared__ __attribute__((aligned(16))) char smem[kSmemBytes];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1;
  const T* __restrict__ hw = static_cast<const T*>(p.hw);
  const T* __restrict__ wd = static_cast<const T*>(p.wd);
  T* __restrict__ o = static_cast<T*>(p.o);
  const int H = p.H, F = p.F;
  const int ntn = H / 128;
  const int total = *p.num_mtiles * ntn;
  const int nk = F / Elem<T>::BK;
  const XcdRange xr = xcd_range(total);
  const int brow[4] = {wn * 64, wn * 64 + 16, wn * 64 + 32, wn * 64 + 48};
  for (int tile = xr.first; tile < xr.end; tile += xr.stride) {
    const int mt = tile / ntn, nt = tile - mt * ntn;
    const int2 me = p.mtile[mt];
    const int e = me.x, r0 = me.y;
    const int seg_end = p.offsets[e + 1];
    KLoader<128> la, lb;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = (tid >> 3) + 32 * i;
      const int r = r0 + row;
      la.p[i] = r < seg_end ? reinterpret_cast<const char*>(hw + (size_t)r * F) + (tid & 7) * 16 : nullptr;
      lb.p[i] = reinterpret_cast<const char*>(wd + ((size_t)e * H + nt * 128 + row) * F) + (tid & 7) * 16;
    }
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
          o[(size_t)r * H + n] = cvt_out<T>(acc[i][j][q]);
        }
      }
    }
  }
}

// out[t] = sum over j with pair_pos[t*k+j] >= 0 of src[pair_pos[t*k+j]]; fp32 accumulation in
// slot order. A token with no local slot gets zeros. One wavefront per part of a row (128 chunks of
// 16 bytes: 2048 bf16) of tpw consecutive tokens (combine_tpw), 4 wavefronts per block (the parts of
// a token in neighbouring wavefronts); the slots' pair positions reach every lane through readlane.
// (One wavefront per whole token left the last of its ~3 rounds of waves per CU mostly empty.)
template <class T>
__global__ __launch_bounds__(256) void k_combine(const T* __restrict__ src, const int* __restrict__ pair_pos,
                                                 T* __restrict__ out, int64_t ntok, int k, int H, int tpw) {
  constexpr int VEC = Elem<T>::VEC;
  const int lane = threadIdx.x & 63;
  const int nch = H / VEC, nparts = (nch + 127) / 128;
  const int64_t u = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t tg = u / nparts;
  const int part = (int)(u - tg * nparts);
  const int64_t t0 = tg * tpw;
  if (t0 >= ntok) return;   // the whole wave leaves
  const int nt = (int)min((int64_t)tpw, ntok - t0);
  const int ppv = lane < nt * k ? pair_pos[t0 * k + lane] : -1;
  for (int tt = 0; tt < nt; ++tt)
    combine_row_part<T, VEC>(src, ppv, tt * k, k, H, nch, part, nparts, lane, out + (t0 + tt) * H);
}

template <class T>
hipError_t launch_forward_gemms(const FwdParams& p, int grid, hipStream_t s, bool recompute) {
  hipError_t err;
  prof_mark_begin(recompute ? "gemm_gateup_recompute" : "gemm_gateup_swiglu", s);
  k_gateup<T><<<grid, kThreads, 0, s>>>(p);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  prof_mark_end(s);
  if (recompute) return hipSuccess;
  prof_mark_begin("gemm_down", s);
  k_down<T><<<grid, kThreads, 0, s>>>(p);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  prof_mark_end(s);
  return hipSuccess;
}

template <class T>
hipError_t launch_combine(const void* src, const int* pair_pos, void* out, int64_t T_, int k, int H, int tpw,
                          hipStream_t s) {
  prof_mark_begin("combine", s);
  const int64_t nparts = (H / Elem<T>::VEC + 127) / 128;
  const int64_t waves = (T_ + tpw - 1) / tpw * nparts;
  k_combine<T><<<(unsigned)((waves + 3) / 4), 256, 0, s>>>(static_cast<const T*>(src), pair_pos,
                                                           static_cast<T*>(out), T_, k, H, tpw);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  prof_mark_end(s);
  return hipSuccess;
}

// Router projection in the fp32 test mode: plain fp32 sums, one thread per output, in a fixed order
// (performance is not the point of this mode; the bf16 engine has the MFMA form).
//   logits[t][e]  = sum_h x[t][h] W_r[e][h]
//   dW_r[e][h]    = sum_t dlogits[t][e] x[t][h]
//   dx[t][h]     += sum_e dlogits[t][e] W_r[e][h]
__global__ __launch_bounds__(256) void k_router_fwd_f32(RouterParams p) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= p.T * p.E) return;
  const int64_t t = i / p.E, e = i - t * p.E;
  const float* x = static_cast<const float*>(p.x) + t * p.H;
  const float* w = static_cast<const float*>(p.wr) + e * p.H;
  float v = 0.f;
  for (int h = 0; h < p.H; ++h) v = fmaf(x[h], w[h], v);
  p.logits[i] = v;
}

__global__ __launch_bounds__(256) void k_router_dw_f32(RouterParams p) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)p.E * p.H) return;
  const int64_t e = i / p.H, h = i - e * p.H;
  const float* x = static_cast<const float*>(p.x);
  float v = 0.f;
  for (int64_t t = 0; t < p.T; ++t) v = fmaf(p.dlogits[t * p.E + e], x[t * p.H + h], v);
  static_cast<float*>(p.dwr)[i] = v;
}

__global__ __launch_bounds__(256) void k_router_dx_f32(RouterParams p) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= p.T * p.H) return;
  const int64_t t = i / p.H, h = i - t * p.H;
  const float* w = static_cast<const float*>(p.wr);
  float v = 0.f;
  for (int e = 0; e < p.E; ++e) v = fmaf(p.dlogits[t * p.E + e], w[(int64_t)e * p.H + h], v);
  static_cast<float*>(p.dx)[i] += v;
}

hipError_t launch_router_fwd_f32(const RouterParams& p, hipStream_t s) {
  prof_mark_begin("router_fwd_f32", s);
  k_router_fwd_f32<<<(unsigned)((p.T * p.E + 255) / 256), 256, 0, s>>>(p);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  prof_mark_end(s);
  return hipSuccess;
}

hipError_t launch_router_bwd_f32(const RouterParams& p, hipStream_t s) {
  hipError_t err;
  prof_mark_begin("router_dw_f32", s);
  k_router_dw_f32<<<(unsigned)(((int64_t)p.E * p.H + 255) / 256), 256, 0, s>>>(p);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  prof_mark_end(s);
  prof_mark_begin("router_dx_f32", s);
  k_router_dx_f32<<<(unsigned)((p.T * p.H + 255) / 256), 256, 0, s>>>(p);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  prof_mark_end(s);
  return hipSuccess;
}

template hipError_t launch_forward_gemms<float>(const FwdParams&, int, hipStream_t, bool);
template hipError_t launch_combine<float>(const void*, const int*, void*, int64_t, int, int, int, hipStream_t);
template hipError_t launch_combine<bf16>(const void*, const int*, void*, int64_t, int, int, int, hipStream_t);

}  // namespace moe
