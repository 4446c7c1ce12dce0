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
// formula gives for them too. v * 2^-s is exact: scaling by a power of two only moves the exponent
// (|v| 2^-s < 512).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_device.h"

namespace moe {

__device__ __forceinline__ int mx_exponent(float amax) {
  const int be = (int)((__float_as_uint(amax) >> 23) & 0xffu);
  return max(be - 127 - 8, -127);   // finite amax has be <= 254, so s <= 119
}

// The element encoding of a block with exponent s, on the hardware's scaled convert
// (v_cvt_scalef32_pk_fp8_f32), which divides by its scale operand 2^s and rounds to nearest even. It
// turns magnitudes of 464 2^s or more into NaN, so values are first clamped to +-448 2^s, in the
// input's units (448 2^s is exact in fp32 for every s). One clamp and half a convert per element,
// where scaling first took a multiply more. The quantiser tests hold it to the oracle's encoding byte
// for byte, over block magnitudes 2^-140 .. 2^120 (subnormal blocks: s = -127), zero blocks and
// saturating blocks.
struct MxScale {
  float up;    // 2^s; 2^-127 is the subnormal 0x00400000
  float lim;   // 448 2^s
};
__device__ __forceinline__ MxScale mx_scale(int s) {
  const float up = s > -127 ? __uint_as_float((unsigned)(127 + s) << 23) : __uint_as_float(0x00400000u);
  return {up, 448.f * up};
}

// the median of v, -lim and lim: one v_med3_f32
__device__ __forceinline__ float mx_clamp(float v, const MxScale& c) { return __builtin_amdgcn_fmed3f(v, -c.lim, c.lim); }

// four fp32 values of a block -> four E4M3 bytes, first value in the low byte
__device__ __forceinline__ unsigned mx_cvt4(float a, float b, float c, float d, const MxScale& sc) {
  typedef short v2s __attribute__((ext_vector_type(2)));
  v2s o = {0, 0};
  o = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(o, mx_clamp(a, sc), mx_clamp(b, sc), sc.up, false);
  o = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(o, mx_clamp(c, sc), mx_clamp(d, sc), sc.up, true);
  return __builtin_bit_cast(unsigned, o);
}

__device__ __forceinline__ uint2 mx_encode8(const float (&v)[8], int s) {
  const MxScale sc = mx_scale(s);
  return make_uint2(mx_cvt4(v[0], v[1], v[2], v[3], sc), mx_cvt4(v[4], v[5], v[6], v[7], sc));
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
  return quad_max(m);
}

// Largest magnitude of a block of 128 held as 8 values by each of 16 consecutive lanes.
// Every lane of the wave must execute it.
__device__ __forceinline__ float mx_amax_x16(const float (&v)[8]) {
  float m = mx_amax_x4(v);
  m = fmaxf(m, dpp_mov<kDppHalfMirror>(m));   // the quads of the group hold their maxima
  m = fmaxf(m, dpp_mov<kDppMirror>(m));
  return m;
}

template <bool BLK>
__device__ __forceinline__ float block_amax(const float (&v)[8]) {
  return BLK ? mx_amax_x16(v) : mx_amax_x4(v);
}

// Scale bytes of the pair-contiguous transposed copies ([nr][Q] fp8, blocks of 32 along the pairs):
// stored K-tile-major, [Q/128][nr][4], so that the 4 bytes of a row's 128-pair K-tile form one dword
// and a tile's rows are contiguous. A producer that covers 128 pairs of a few rows then writes whole
// lines (a [nr][Q/32] layout gave each line of scales 4-byte runs from 32 different tiles). Offset
// of the byte for row r, pair column q:
__device__ __forceinline__ size_t tscale_at(int64_t nr, int64_t r, int64_t q) {
  return (size_t)(((q >> 7) * nr + r) * 4 + ((q >> 5) & 3));
}

}  // namespace moe
