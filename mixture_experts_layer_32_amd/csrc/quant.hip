// MXFP8 quantisation of the GEMM operands that are not produced by a GEMM epilogue. Every output is
// K-major (the contraction axis contiguous), with its e8m0 scales in a [rows][K/32] byte array, so
// that the fp8 GEMMs read both operands the same way.
//
//   k_quant_rows      along the contiguous axis: x and dY rows (along H), W_gate and W_up rows
//                     (along H), W_down rows (along F), and the transposed hw copy (along pairs).
//                     One lane per 8 elements; 4 lanes per block of 32.
//   k_quant_cols      along the strided axis, transposing: W_down[e] (H x F) along H into F x H,
//                     and W_gate[e], W_up[e] (F x H) along F into the two halves of H x 2F.
//   k_gather_t_quant  along an expert's pairs, transposing and gathering: dY and x rows of the
//                     expert's tokens, in the sorted pair order, into [H][Q] where the expert's
//                     pairs occupy columns qoff[e] .. qoff[e+1] (zero-padded to a multiple of 64).
// The quantised element and scale formulas are in mx_device.h.
#include "moe_device.h"
#include "moe_internal.h"
#include "mx_device.h"

namespace moe {
namespace {

__device__ __forceinline__ void unpack8f(uint4 u, float (&v)[8]) {
  const bf16x8 b = __builtin_bit_cast(bf16x8, u);
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = (float)b[e];
}

// n8 = elements / 8 (a multiple of 4: blocks never straddle a thread group)
__global__ __launch_bounds__(256) void k_quant_rows(const bf16* __restrict__ in, uint8_t* __restrict__ q,
                                                    uint8_t* __restrict__ sc, int64_t n8) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  float v[8];
  if (i < n8) {
    unpack8f(ld16(in + i * 8), v);
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = 0.f;
  }
  const int s = mx_exponent(mx_amax_x4(v));
  if (i < n8) {
    *reinterpret_cast<uint2*>(q + i * 8) = mx_encode8(v, s);
    if ((i & 3) == 0) sc[i >> 2] = (uint8_t)(s + 127);
  }
}

// Column pass shared by the transposing kernels: the block's LDS tile holds 64 source rows of 128
// columns (bf16). Thread t quantises column t & 127 over rows 32 (t >> 7) .. +31 into 32 output
// bytes at out_row + 32 (t >> 7) and one scale byte at sc_row + (t >> 7).
__device__ __forceinline__ void column_pass(const bf16 (*tile)[128], uint8_t* out_row, uint8_t* sc_row) {
  const int c = threadIdx.x & 127, half = threadIdx.x >> 7;
  float v[32];
  float m = 0.f;
#pragma unroll
  for (int r = 0; r < 32; ++r) {
    v[r] = (float)tile[32 * half + r][c];
    m = fmaxf(m, fabsf(v[r]));
  }
  const int s = mx_exponent(m);
  const float sm = mx_inv_scale(s);
  unsigned w[8];
#pragma unroll
  for (int g = 0; g < 8; ++g)
    w[g] = mx_cvt4(mx_sat(v[4 * g] * sm), mx_sat(v[4 * g + 1] * sm), mx_sat(v[4 * g + 2] * sm), mx_sat(v[4 * g + 3] * sm));
  uint4* o = reinterpret_cast<uint4*>(out_row + 32 * half);
  o[0] = make_uint4(w[0], w[1], w[2], w[3]);
  o[1] = make_uint4(w[4], w[5], w[6], w[7]);
  sc_row[half] = (uint8_t)(s + 127);
}

// in [B][R][C] -> out[b][c][col0 + r] (row stride ldo bytes), scales [b][c][(col0 + r) / 32]
// (row stride ldo / 32). Grid (C / 128, R / 64, B).
__global__ __launch_bounds__(256) void k_quant_cols(const bf16* __restrict__ in, uint8_t* __restrict__ q,
                                                    uint8_t* __restrict__ sc, int R, int C, int64_t ldo, int col0) {
  __shared__ __attribute__((aligned(16))) bf16 tile[64][128];
  const int b = blockIdx.z, r0 = blockIdx.y * 64, c0 = blockIdx.x * 128, t = threadIdx.x;
  const bf16* src = in + ((size_t)b * R + r0) * C + c0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int ch = t + 256 * i, row = ch >> 4, c8 = (ch & 15) * 8;
    *reinterpret_cast<uint4*>(&tile[row][c8]) = ld16(src + (size_t)row * C + c8);
  }
  __syncthreads();
  const size_t orow = (size_t)b * C + c0 + (t & 127);
  column_pass(tile, q + orow * ldo + col0 + r0, sc + orow * (ldo / 32) + (col0 + r0) / 32);
}

// Grid (qc / 64, H / 128). Window w covers columns 64w .. 64w+63 of [H][qc], inside one expert's
// padded segment.
__global__ __launch_bounds__(256) void k_gather_t_quant(const bf16* __restrict__ x, const int* __restrict__ ptok,
                                                        const int* __restrict__ offsets, const int* __restrict__ qoff,
                                                        int El, int H, int64_t qc, uint8_t* __restrict__ q,
                                                        uint8_t* __restrict__ sc) {
  __shared__ __attribute__((aligned(16))) bf16 tile[64][128];
  const int q0 = blockIdx.x * 64, h0 = blockIdx.y * 128, t = threadIdx.x;
  if (q0 >= qoff[El]) return;   // past the last expert's segment: nothing reads these columns
  int lo = 0, hi = El - 1;      // the expert whose segment holds q0: the last e with qoff[e] <= q0
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (qoff[mid] <= q0) lo = mid;
    else hi = mid - 1;
  }
  const int base = offsets[lo] + (q0 - qoff[lo]), end = offsets[lo + 1];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int ch = t + 256 * i, row = ch >> 4, c8 = (ch & 15) * 8;
    const int r = base + row;
    *reinterpret_cast<uint4*>(&tile[row][c8]) =
        r < end ? ld16(x + (size_t)ptok[r] * H + h0 + c8) : make_uint4(0u, 0u, 0u, 0u);
  }
  __syncthreads();
  const size_t orow = (size_t)h0 + (t & 127);
  column_pass(tile, q + orow * qc + q0, sc + orow * (qc / 32) + q0 / 32);
}

}  // namespace

hipError_t launch_quant_rows(const void* in, uint8_t* q, uint8_t* sc, int64_t n, const char* name, hipStream_t s) {
  const int64_t n8 = n / 8;
  prof_mark_begin(name, s);
  k_quant_rows<<<(unsigned)((n8 + 255) / 256), 256, 0, s>>>(static_cast<const bf16*>(in), q, sc, n8);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  prof_mark_end(s);
  return hipSuccess;
}

hipError_t launch_quant_cols(const void* in, uint8_t* q, uint8_t* sc, int B, int R, int C, int64_t ldo, int col0,
                             const char* name, hipStream_t s) {
  prof_mark_begin(name, s);
  k_quant_cols<<<dim3(C / 128, R / 64, B), 256, 0, s>>>(static_cast<const bf16*>(in), q, sc, R, C, ldo, col0);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  prof_mark_end(s);
  return hipSuccess;
}

hipError_t launch_gather_t_quant(const void* x, const int* ptok, const int* offsets, const int* qoff, int El, int H,
                                 int64_t qc, uint8_t* q, uint8_t* sc, const char* name, hipStream_t s) {
  prof_mark_begin(name, s);
  k_gather_t_quant<<<dim3((unsigned)(qc / 64), H / 128), 256, 0, s>>>(static_cast<const bf16*>(x), ptok, offsets,
                                                                     qoff, El, H, qc, q, sc);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  prof_mark_end(s);
  return hipSuccess;
}

}  // namespace moe
