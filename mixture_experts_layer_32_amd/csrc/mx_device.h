// MXFP8 encoding on gfx950. The precision mode is named in "Supporto di precisione e vincoli
// hardware" on "Prime Mega MoE: il kernel che accelera il training AI del 55%". The pages give no
// format details; the library reads it as the OCP microscaling format:
//  * 32 consecutive elements along a GEMM's contraction axis share one scale 2^s, stored as the
//    e8m0 byte s + 127;
//  * s = floor(log2 amax) - 8 (8 is the exponent of E4M3's largest normal), clamped to
//    [-127, 127], so an all-zero block gets s = -127;
//  * elements are E4M3 (finite-only form, largest value 448) of v * 2^-s, rounded to nearest
//    even and saturated to +-448.
// floor(log2 amax) of a normal fp32 amax is its biased exponent minus 127. Zero and subnormal amax
// (below 2^-126) give biased exponent 0, and the clamp then yields -127, which is the value the
// formula gives for them too. v * 2^-s is exact in fp32: the power of two is a normal number and
// |v| 2^-s < 512. The hardware convert rounds to nearest even, but it turns values of magnitude
// 464 or more into NaN, so values are clamped to +-448 before it.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

__device__ __forceinline__ int mx_exponent(float amax) {
  const int be = (int)((__float_as_uint(amax) >> 23) & 0xffu);
  return max(be - 127 - 8, -127);   // finite amax has be <= 254, so s <= 119
}

// 2^-s for s in [-127, 119]: biased exponent 127 - s lies in [8, 254]
__device__ __forceinline__ float mx_inv_scale(int s) { return __uint_as_float((unsigned)(127 - s) << 23); }

__device__ __forceinline__ float mx_sat(float v) { return fminf(fmaxf(v, -448.f), 448.f); }

// four fp32 values (already scaled and saturated) -> four E4M3 bytes, first value in the low byte
__device__ __forceinline__ unsigned mx_cvt4(float a, float b, float c, float d) {
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return (unsigned)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true);
}

__device__ __forceinline__ uint2 mx_encode8(const float (&v)[8], int s) {
  const float m = mx_inv_scale(s);
  return make_uint2(mx_cvt4(mx_sat(v[0] * m), mx_sat(v[1] * m), mx_sat(v[2] * m), mx_sat(v[3] * m)),
                    mx_cvt4(mx_sat(v[4] * m), mx_sat(v[5] * m), mx_sat(v[6] * m), mx_sat(v[7] * m)));
}

// Blockwise FP8 (the FP8 mode; the same pages list a blockwise-scaled FP8 without block sizes). The
// library reads it with power-of-two scales, the form the scaled MFMA consumes: the scale of a block
// is the smallest 2^s with amax <= 448 * 2^s, s clamped to [-127, 127], so no element saturates.
// With amax = m 2^e (m in [1, 2)), 448 2^(e-8) = 1.75 2^e: s = e - 8, plus one when m > 1.75, i.e.
// when the fp32 mantissa field exceeds 0x600000. Zero and subnormal amax give s = -127.
__device__ __forceinline__ int fp8b_exponent(float amax) {
  const unsigned u = __float_as_uint(amax);
  const int be = (int)((u >> 23) & 0xffu);
  return max(be - 127 - 8 + ((u & 0x7fffffu) > 0x600000u ? 1 : 0), -127);
}

template <bool BLK>
__device__ __forceinline__ int block_exponent(float amax) {
  return BLK ? fp8b_exponent(amax) : mx_exponent(amax);
}

// Largest magnitude of a block of 32 held as 8 values by each of 4 consecutive lanes (lanes 4g..4g+3).
// Every lane of the wave must execute it.
__device__ __forceinline__ float mx_amax_x4(const float (&v)[8]) {
  float m = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf(v[e]));
  m = fmaxf(m, __shfl_xor(m, 1));
  m = fmaxf(m, __shfl_xor(m, 2));
  return m;
}

// Largest magnitude of a block of 128 held as 8 values by each of 16 consecutive lanes.
// Every lane of the wave must execute it.
__device__ __forceinline__ float mx_amax_x16(const float (&v)[8]) {
  float m = mx_amax_x4(v);
  m = fmaxf(m, __shfl_xor(m, 4));
  m = fmaxf(m, __shfl_xor(m, 8));
  return m;
}

template <bool BLK>
__device__ __forceinline__ float block_amax(const float (&v)[8]) {
  return BLK ? mx_amax_x16(v) : mx_amax_x4(v);
}

}  // namespace moe
