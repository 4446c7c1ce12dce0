// MXFP8 quantisation of the GEMM operands that are not produced by a GEMM epilogue. Every output is
// K-major (the contraction axis contiguous), with its e8m0 scales in a [rows][K/32] byte array
// (the pair-contiguous copies: [K/128][rows][4]), so that the fp8 GEMMs read both operands the same
// way.
//
//   k_quant_rows      along the contiguous axis: x and dY rows (along H), W_gate and W_up rows
//                     (along H), W_down rows (along F), and the transposed hw copy (along pairs).
//                     One lane per 8 elements; 4 lanes per block of 32.
//   k_quant_cols      along the strided axis, transposing: W_down[e] (H x F) along H into F x H,
//                     and W_gate[e], W_up[e] (F x H) along F into the two halves of H x 2F
//                     (k_quant_cols128 when the column count is a multiple of 128).
//   k_quant_both      both orientations of one weight tensor from one read (the MXFP8 forward
//                     quantises each weight once per step for both passes); 128 x 128 tiles.
//                     Either orientation is skipped when its output is null.
//   k_gather_t_quant  along an expert's pairs, transposing and gathering: dY and x rows of the
//                     expert's tokens, in the sorted pair order, into [H][Q] where the expert's
//                     pairs occupy columns qoff[e] .. qoff[e+1] (zero-padded to a multiple of 128);
//                     its scales are K-tile-major, [Q/128][H][4] (tscale_at).
// The transposing kernels stage 128 x 64 tiles (k_quant_both: 128 x 128) in LDS, so that every
// row segment they read or write is one or two whole 128-byte lines. The weights' scale bytes are
// the exception: a tile writes 4 of them per row of a [rows][K/32] array, so a 128-byte line of
// scales is filled by many blocks. The grids are one-dimensional with consecutive tiles on one XCD
// (xcd_logical_block), so that those blocks meet in one L2, which merges the line before writing
// it back. (The gathered transpose's scales are K-tile-major: a tile's 64 rows x 4 bytes are
// contiguous.)
// The quantised element and scale formulas are in mx_device.h.
//
// Blockwise FP8 (template flag BLK): k_quant_rows takes blocks of 128 along the row (16 lanes),
// k_quant_both one scale per 128 x 128 tile for both orientations, and k_gather_t_quant blocks of
// the 128 pairs of a window. The scale arrays keep the MXFP8 layout (one byte per 32 elements), with
// each block's scale repeated over its 32-element groups, so the fp8 GEMMs read both forms alike.
#include "moe_device.h"
#include "moe_internal.h"
#include "mx_device.h"

namespace moe {
namespace {

// tile (x, y, b) of a grid of nx x ny x B tiles run as a one-dimensional grid: logical tile ids, x
// fastest, then y, then b, in contiguous ranges per XCD
struct Tile3 {
  int x, y, b;
};
__device__ __forceinline__ Tile3 tile_of_block(int nx, int ny) {
  const int n = xcd_logical_block(gridDim.x);
  Tile3 t;
  t.x = n % nx;
  t.y = (n / nx) % ny;
  t.b = n / (nx * ny);
  return t;
}

__device__ __forceinline__ void unpack8f(uint4 u, float (&v)[8]) {
  const bf16x8 b = __builtin_bit_cast(bf16x8, u);
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = (float)b[e];
}

// n8 = elements / 8 (a multiple of 4, of 16 with BLK: blocks never straddle a thread group)
template <bool BLK>
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
  const int s = block_exponent<BLK>(block_amax<BLK>(v));
  if (i < n8) {
    *reinterpret_cast<uint2*>(q + i * 8) = mx_encode8(v, s);
    if ((i & 3) == 0) sc[i >> 2] = (uint8_t)(s + 127);
  }
}

// Column pass shared by the transposing kernels: the block's LDS tile holds 128 source rows of 64
// columns (bf16). Thread t quantises column t & 63 over rows 32 (t >> 6) .. +31 into 32 output
// bytes at out_row + 32 (t >> 6) and one scale byte at sc_row + (t >> 6). The four threads of a
// column write one whole 128-byte line. With BLK the column's 128 rows are one block: the four
// threads (one per wave) exchange their maxima through cmax [4][64] (a barrier every thread reaches).
template <bool BLK>
__device__ __forceinline__ void column_pass(const bf16 (*tile)[64], uint8_t* out_row, uint8_t* sc_row, float* cmax) {
  const int c = threadIdx.x & 63, blk = threadIdx.x >> 6;
  float v[32];
  float m = 0.f;
#pragma unroll
  for (int r = 0; r < 32; ++r) {
    v[r] = (float)tile[32 * blk + r][c];
    m = fmaxf(m, fabsf(v[r]));
  }
  if constexpr (BLK) {
    cmax[threadIdx.x] = m;
    __syncthreads();
    m = fmaxf(fmaxf(cmax[c], cmax[64 + c]), fmaxf(cmax[128 + c], cmax[192 + c]));
  }
  const int s = block_exponent<BLK>(m);
  const MxScale sc = mx_scale(s);
  unsigned w[8];
#pragma unroll
  for (int g = 0; g < 8; ++g) w[g] = mx_cvt4(v[4 * g], v[4 * g + 1], v[4 * g + 2], v[4 * g + 3], sc);
  uint4* o = reinterpret_cast<uint4*>(out_row + 32 * blk);
  o[0] = make_uint4(w[0], w[1], w[2], w[3]);
  o[1] = make_uint4(w[4], w[5], w[6], w[7]);
  sc_row[blk] = (uint8_t)(s + 127);
}

// Loads rows r0..r0+127, columns c0..c0+63 of a row-major bf16 matrix (row pointers from row_ptr)
// into the LDS tile: 8 lanes per row, one whole 128-byte line each. Load i of thread t covers row
// (t >> 3) + 32i, columns 8 (t & 7) .. +7, and is also returned in raw[i].
template <class RowPtr>
__device__ __forceinline__ void load_tile(bf16 (*tile)[64], RowPtr row_ptr, uint4 (&raw)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int ch = threadIdx.x + 256 * i, row = ch >> 3, c8 = (ch & 7) * 8;
    const bf16* src = row_ptr(row);
    raw[i] = src ? ld16(src + c8) : make_uint4(0u, 0u, 0u, 0u);
    *reinterpret_cast<uint4*>(&tile[row][c8]) = raw[i];
  }
}

// in [B][R][C] -> out[b][c][col0 + r] (row stride ldo bytes), scales [b][c][(col0 + r) / 32]
// (row stride ldo / 32). Tiles (C / 64, R / 128, B).
__global__ __launch_bounds__(256) void k_quant_cols(const bf16* __restrict__ in, uint8_t* __restrict__ q,
                                                    uint8_t* __restrict__ sc, int R, int C, int64_t ldo, int col0) {
  __shared__ __attribute__((aligned(16))) bf16 tile[128][64];
  const Tile3 tt = tile_of_block(C / 64, R / 128);
  const int b = tt.b, r0 = tt.y * 128, c0 = tt.x * 64;
  const bf16* src = in + ((size_t)b * R + r0) * C + c0;
  uint4 raw[4];
  load_tile(tile, [&](int row) { return src + (size_t)row * C; }, raw);
  __syncthreads();
  const size_t orow = (size_t)b * C + c0 + (threadIdx.x & 63);
  column_pass<false>(tile, q + orow * ldo + col0 + r0, sc + orow * (ldo / 32) + (col0 + r0) / 32, nullptr);
}

// Column pass on a 128 x 128 LDS tile: thread t quantises column t & 127 over the blocks of 32 rows
// 2 (t >> 7) and 2 (t >> 7) + 1, into the 32-byte segments out_row + 32 blk and the scale bytes
// sc_row[blk]. The two threads of a column write one whole 128-byte line. With BLK every block takes
// the tile's exponent s_tile.
template <bool BLK>
__device__ __forceinline__ void column_pass128(const bf16 (*tile)[128], uint8_t* out_row, uint8_t* sc_row,
                                               int s_tile) {
  const int t = threadIdx.x, c = t & 127;
#pragma unroll
  for (int bb = 0; bb < 2; ++bb) {
    const int blk = 2 * (t >> 7) + bb;
    float v[32];
    float m = 0.f;
#pragma unroll
    for (int r = 0; r < 32; ++r) {
      v[r] = (float)tile[32 * blk + r][c];
      m = fmaxf(m, fabsf(v[r]));
    }
    const int s = BLK ? s_tile : mx_exponent(m);
    const MxScale sc = mx_scale(s);
    unsigned w[8];
#pragma unroll
    for (int g = 0; g < 8; ++g) w[g] = mx_cvt4(v[4 * g], v[4 * g + 1], v[4 * g + 2], v[4 * g + 3], sc);
    st16(out_row + 32 * blk, make_uint4(w[0], w[1], w[2], w[3]));
    st16(out_row + 32 * blk + 16, make_uint4(w[4], w[5], w[6], w[7]));
    sc_row[blk] = (uint8_t)(s + 127);
  }
}

// As k_quant_cols on 128 x 128 tiles (C a multiple of 128): tiles (C / 128, R / 128, B). The two
// threads of a column write one whole 128-byte line; the input is read once (non-temporal loads).
__global__ __launch_bounds__(256) void k_quant_cols128(const bf16* __restrict__ in, uint8_t* __restrict__ q,
                                                       uint8_t* __restrict__ sc, int R, int C, int64_t ldo, int col0) {
  __shared__ __attribute__((aligned(16))) bf16 tile[128][128];
  const Tile3 tt = tile_of_block(C / 128, R / 128);
  const int t = threadIdx.x, b = tt.b, r0 = tt.y * 128, c0 = tt.x * 128;
  const bf16* src = in + ((size_t)b * R + r0) * C + c0;
  const int col8 = (t & 15) * 8;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int row = (t >> 4) + 16 * i;
    *reinterpret_cast<uint4*>(&tile[row][col8]) = ld16_nt(src + (size_t)row * C + col8);
  }
  __syncthreads();
  const size_t orow = (size_t)b * C + c0 + (t & 127);
  column_pass128<false>(tile, q + orow * ldo + col0 + r0, sc + orow * (ldo / 32) + (col0 + r0) / 32, 0);
}

// Both orientations of one weight tensor in one read: in [B][R][C] ->
//   rows: qr [B][R][C] with blocks of 32 along C, scales sr [B][R][C/32]
//   cols: blocks of 32 along R, written transposed at column col0 of rows of ldo bytes:
//         qc [B][C][ldo], scales scc [B][C][ldo/32]
// Tiles (C / 128, R / 128, B). A block stages a 128 x 128 bf16 tile (32 KB), so that the row pass
// writes whole 128-byte lines of fp8 (16 lanes per row, quantised from the registers that loaded
// the tile) and the column pass too (each thread quantises two blocks of 32 of one column). The
// input is read once: non-temporal loads. The stores stay ordinary: each instruction writes less
// than a whole line per row, and non-temporal partial-line stores ran 3.4x slower.
// BLK: one exponent for the whole tile (its amax over the 4 waves), in both orientations.
template <bool BLK>
__global__ __launch_bounds__(256) void k_quant_both(const bf16* __restrict__ in, uint8_t* __restrict__ qr,
                                                    uint8_t* __restrict__ sr, uint8_t* __restrict__ qc,
                                                    uint8_t* __restrict__ scc, int R, int C, int64_t ldo, int col0) {
  __shared__ __attribute__((aligned(16))) bf16 tile[128][128];
  const Tile3 tt = tile_of_block(C / 128, R / 128);
  const int t = threadIdx.x, b = tt.b, r0 = tt.y * 128, c0 = tt.x * 128;
  const bf16* src = in + ((size_t)b * R + r0) * C + c0;
  const int col8 = (t & 15) * 8;
  uint4 raw[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int row = (t >> 4) + 16 * i;
    raw[i] = ld16_nt(src + (size_t)row * C + col8);
    *reinterpret_cast<uint4*>(&tile[row][col8]) = raw[i];
  }
  int s_tile = 0;
  if constexpr (BLK) {
    __shared__ float wmax[4];
    float m = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float v[8];
      unpack8f(raw[i], v);
#pragma unroll
      for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf(v[e]));
    }
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) m = fmaxf(m, __shfl_xor(m, d));
    if ((t & 63) == 0) wmax[t >> 6] = m;
    __syncthreads();
    s_tile = fp8b_exponent(fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3])));
  }
  // row pass: the 4 lanes 4g..4g+3 hold one row's block of 32 along C (skipped when qr is null)
  if (qr) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float v[8];
      unpack8f(raw[i], v);
      const int s = BLK ? s_tile : mx_exponent(mx_amax_x4(v));
      const size_t grow = (size_t)b * R + r0 + (t >> 4) + 16 * i;
      *reinterpret_cast<uint2*>(qr + grow * C + c0 + col8) = mx_encode8(v, s);
      if ((t & 3) == 0) sr[grow * (C / 32) + (c0 + col8) / 32] = (uint8_t)(s + 127);
    }
  }
  if (!qc) return;   // no column pass (the whole block takes this branch)
  __syncthreads();
  const size_t orow = (size_t)b * C + c0 + (t & 127);
  column_pass128<BLK>(tile, qc + orow * ldo + col0 + r0, scc + orow * (ldo / 32) + (col0 + r0) / 32, s_tile);
}

// Blocks (window w, split s) for w < qc / 128, s < GT_SPLIT, logical id GT_SPLIT w + s. Window w
// covers columns 128w .. 128w+127 of [H][qc], inside one expert's padded segment (segments are
// multiples of 128 columns). A block finds its expert and the window's 128 token indices once, then
// walks the 64-column tiles h0 = 64 (s + GT_SPLIT j) of H: the next tile's rows load while the
// current one is quantised. A window's splits run side by side on one XCD, reading neighbouring
// 128-byte segments of the same rows (6-7 % faster than splits in separate ranges, and than 4 or
// 2 splits; 16 measured the same as 8). 128 x 128 tiles measured 10-15 % slower here.
constexpr int GT_SPLIT = 8;
template <bool BLK>
__global__ __launch_bounds__(256) void k_gather_t_quant(const bf16* __restrict__ x, const int* __restrict__ ptok,
                                                        const int* __restrict__ offsets, const int* __restrict__ qoff,
                                                        int El, int H, int64_t qc, uint8_t* __restrict__ q,
                                                        uint8_t* __restrict__ sc) {
  __shared__ __attribute__((aligned(16))) bf16 tile[128][64];
  __shared__ float cmax[BLK ? 256 : 1];
  const int n = xcd_logical_block(gridDim.x), split = n % GT_SPLIT;
  const int q0 = (n / GT_SPLIT) * 128;
  if (q0 >= qoff[El]) return;   // past the last expert's segment: nothing reads these columns
  int lo = 0, hi = El - 1;      // the expert whose segment holds q0: the last e with qoff[e] <= q0
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (qoff[mid] <= q0) lo = mid;
    else hi = mid - 1;
  }
  const int base = offsets[lo] + (q0 - qoff[lo]), end = offsets[lo + 1];
  // load i of this thread covers tile row (t >> 3) + 32 i, columns 8 (t & 7) .. +7
  const bf16* src[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = (threadIdx.x >> 3) + 32 * i;
    src[i] = base + row < end ? x + (size_t)ptok[base + row] * H + (threadIdx.x & 7) * 8 : nullptr;
  }
  auto load = [&](int h0, uint4 (&raw)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) raw[i] = src[i] ? ld16(src[i] + h0) : make_uint4(0u, 0u, 0u, 0u);
  };
  uint4 raw[4], nxt[4];
  int h0 = 64 * split;
  if (h0 >= H) return;
  load(h0, nxt);
  for (; h0 < H; h0 += 64 * GT_SPLIT) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      raw[i] = nxt[i];
      *reinterpret_cast<uint4*>(&tile[(threadIdx.x >> 3) + 32 * i][(threadIdx.x & 7) * 8]) = raw[i];
    }
    __syncthreads();
    if (h0 + 64 * GT_SPLIT < H) load(h0 + 64 * GT_SPLIT, nxt);
    const size_t orow = (size_t)h0 + (threadIdx.x & 63);
    column_pass<BLK>(tile, q + orow * qc + q0, sc + tscale_at(H, orow, q0), cmax);
    __syncthreads();   // the tile (and cmax) are overwritten next
  }
}

}  // namespace

hipError_t launch_quant_rows(const void* in, uint8_t* q, uint8_t* sc, int64_t n, const char* name, hipStream_t s,
                             bool blk) {
  const int64_t n8 = n / 8;
  prof_mark_begin(name, s);
  if (blk)
    k_quant_rows<true><<<(unsigned)((n8 + 255) / 256), 256, 0, s>>>(static_cast<const bf16*>(in), q, sc, n8);
  else
    k_quant_rows<false><<<(unsigned)((n8 + 255) / 256), 256, 0, s>>>(static_cast<const bf16*>(in), q, sc, n8);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  prof_mark_end(s);
  return hipSuccess;
}

hipError_t launch_quant_cols(const void* in, uint8_t* q, uint8_t* sc, int B, int R, int C, int64_t ldo, int col0,
                             const char* name, hipStream_t s) {
  prof_mark_begin(name, s);
  if (C % 128 == 0)
    k_quant_cols128<<<(C / 128) * (R / 128) * B, 256, 0, s>>>(static_cast<const bf16*>(in), q, sc, R, C, ldo, col0);
  else
    k_quant_cols<<<(C / 64) * (R / 128) * B, 256, 0, s>>>(static_cast<const bf16*>(in), q, sc, R, C, ldo, col0);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  prof_mark_end(s);
  return hipSuccess;
}

hipError_t launch_quant_both(const void* in, uint8_t* qr, uint8_t* sr, uint8_t* qc, uint8_t* scc, int B, int R, int C,
                             int64_t ldo, int col0, const char* name, hipStream_t s, bool blk) {
  prof_mark_begin(name, s);
  const unsigned grid = (C / 128) * (R / 128) * B;
  if (blk)
    k_quant_both<true><<<grid, 256, 0, s>>>(static_cast<const bf16*>(in), qr, sr, qc, scc, R, C, ldo, col0);
  else
    k_quant_both<false><<<grid, 256, 0, s>>>(static_cast<const bf16*>(in), qr, sr, qc, scc, R, C, ldo, col0);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  prof_mark_end(s);
  return hipSuccess;
}

hipError_t launch_gather_t_quant(const void* x, const int* ptok, const int* offsets, const int* qoff, int El, int H,
                                 int64_t qc, uint8_t* q, uint8_t* sc, const char* name, hipStream_t s, bool blk) {
  prof_mark_begin(name, s);
  const unsigned grid = (unsigned)(qc / 128) * GT_SPLIT;
  if (blk)
    k_gather_t_quant<true><<<grid, 256, 0, s>>>(static_cast<const bf16*>(x), ptok, offsets, qoff, El, H, qc, q, sc);
  else
    k_gather_t_quant<false><<<grid, 256, 0, s>>>(static_cast<const bf16*>(x), ptok, offsets, qoff, El, H, qc, q, sc);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  prof_mark_end(s);
  return hipSuccess;
}

}  // namespace moe
