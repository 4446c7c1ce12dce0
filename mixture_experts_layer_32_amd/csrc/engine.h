// Pieces of the gfx950 grouped-GEMM engine shared by the bf16 and MXFP8 kernels: tile geometry,
// direct-to-LDS loads and their waits, the K-major LDS layout and fragment reads, the K-major operand
// loader, and the LDS-staged epilogue helpers.
//
// Tile geometry: a workgroup computes a 256x256 output tile as 32x32 MFMA output blocks. Each wave
// owns an MI x NJ grid of blocks: with 4 waves a 128x128 quadrant (4x4), with 8 waves a 64x128 or
// 128x64 eighth. Each engine sets its wave count, K-tile (the bytes of contraction per operand row)
// and ring depth. The operand tiles of a K-tile reach LDS with global_load_lds_dwordx4.
#pragma once
#include "moe_device.h"
#include "mx_device.h"

namespace moe {
namespace eng {

typedef __attribute__((address_space(3))) void lds_t;
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

constexpr int TILE = 256;            // output tile rows and columns
constexpr int NTHR = 256;            // threads of a 4-wave workgroup

// One wave-wide direct-to-LDS load: lane i copies 16 bytes from g into lds + 16*i (lds is
// wave-uniform). Written as inline assembly so that the compiler neither tracks it nor inserts
// waits for it. The main loop orders these loads with explicit vmcnt waits and barriers.
__device__ __forceinline__ void gl2lds(const void* g, char* lds) {
  // the LDS address: the low 32 bits of a generic pointer into the LDS aperture (a cast to the LDS
  // address space would add a null check, which needs the aperture's high half in a register)
  const unsigned off = __builtin_amdgcn_readfirstlane((unsigned)(uintptr_t)lds);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(off), "v"(g) : "memory", "m0");
}
// wait until at most N vector memory operations of this wave are outstanding
template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
// workgroup barrier without a memory fence. The caller has already waited for the loads the
// barrier publishes; lgkmcnt(0) retires this wave's LDS reads before other waves may overwrite
// the stage.
__device__ __forceinline__ void block_sync() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }
// p[i] for a wave-uniform i, through the scalar unit. Read through the constant address space, the
// data is known not to change during the kernel, so the compiler emits s_load_dword: the value counts
// against lgkmcnt, not vmcnt. A plain load here becomes a vector load whose compiler-inserted
// vmcnt waits also wait for the direct-to-LDS tile loads in flight, which the compiler does not see.
__device__ __forceinline__ int ld_uniform(const int* p, int i) {
  return ((const __attribute__((address_space(4))) int*)p)[i];
}

// Dynamic tile scheduler of the persistent kernels. The tile list is cut into 8 contiguous ranges,
// one per XCD (workgroups are dispatched to the XCDs round-robin: workgroup b runs on XCD b % 8), so
// that the workgroups sharing an XCD's L2 work on neighbouring tiles, which share operands. Within
// its range, an XCD's workgroups take tiles in order from a counter, one atomic increment per tile,
// so that a workgroup that drew cheaper tiles (an expert's half tile) takes more of them. ctr points
// at the kernel's 8 per-XCD counters, zero at launch. Every thread of the workgroup calls first()
// and next(); both contain a barrier, and return the next tile, or -1 once the range is exhausted.
// Between them the tile's work calls fetch() once, after its main loop (so that the returned
// counter does not occupy a register through the loop, and its latency hides behind the epilogue);
// the work must contain a barrier before next(), which overwrites the LDS slot. Without fetch(),
// next() ends the loop.
struct TileSched {
  int* ctr;
  int begin, end, nxt;
  __device__ __forceinline__ TileSched(int* counters, int total) {
    const int xcd = blockIdx.x & 7, per = (total + 7) >> 3;
    begin = min(total, xcd * per);
    end = min(total, begin + per);
    ctr = counters + xcd;
    nxt = 0;
  }
  __device__ __forceinline__ int take(int t) {
    nxt = end - begin;   // past the range unless fetch() runs
    const int tile = begin + t;
    return tile < end ? tile : -1;
  }
  __device__ __forceinline__ void fetch() {
    if (threadIdx.x == 0) nxt = atomicAdd(ctr, 1);
  }
  __device__ __forceinline__ int first(int* slot) {
    if (threadIdx.x == 0) *slot = atomicAdd(ctr, 1);
    block_sync();
    return take(*slot);
  }
  __device__ __forceinline__ int next(int* slot) {
    if (threadIdx.x == 0) *slot = nxt;
    block_sync();
    return take(*slot);
  }
};

// Static per-XCD tile range whose 9 boundaries b[0..8] were written by a previous kernel (the
// weight-gradient GEMMs' cost-balanced split); within it the XCD's workgroups take tiles round-robin.
__device__ __forceinline__ XcdRange xcd_range_split(const int* b) {
  const int xcd = blockIdx.x & 7;
  XcdRange r;
  r.begin = ld_uniform(b, xcd);
  r.end = ld_uniform(b, xcd + 1);
  r.stride = gridDim.x >> 3;
  r.first = r.begin + (blockIdx.x >> 3);
  return r;
}

// K-major operand of 256 rows with ROWB bytes of contraction per row per K-tile (64 or 128).
// One wave instruction moves RPI = 64/NCH whole row segments (NCH = ROWB/16 chunks of 16 bytes);
// with NW waves sharing the tile, this lane owns rows (w*LOADS + j)*RPI + lane/NCH and slot lane%NCH. A 128-byte segment is a
// whole cache line: the direct-to-LDS path moves twice the bytes per cycle with whole lines as
// with half lines.
// LDS: row r at r*ROWB, chunk c at slot c ^ swz(r). A ds_read_b128 serves 16 lanes per pass over
// the 64 banks (256 bytes). The 16 lanes read 16 consecutive rows at one chunk, and swz spreads
// them over distinct bank groups:
//   64-byte rows:  4 rows share 256 bytes, swz = (r >> 2) & 3
//   128-byte rows: 2 rows share 256 bytes, swz = (r >> 1) & 7
template <int ROWB, int NW = 4>
struct KRows {
  static constexpr int NCH = ROWB / 16, RPI = 64 / NCH, LOADS = TILE / (NW * RPI);
  const char* p[LOADS];   // global address of this lane's chunk in K-tile 0
  __device__ __forceinline__ static int swz(int r) { return ROWB == 64 ? (r >> 2) & 3 : (r >> 1) & 7; }
  __device__ __forceinline__ static int row_of(int j) {
    return (wave_id() * LOADS + j) * RPI + (threadIdx.x & 63) / NCH;
  }
  __device__ __forceinline__ static int chunk_of(int j) { return (threadIdx.x & (NCH - 1)) ^ swz(row_of(j)); }
  __device__ __forceinline__ void prefetch(int) {}
  __device__ __forceinline__ void prologue_prefetch(int) {}
  __device__ __forceinline__ void prologue_issue(char* tile, int kt) const { issue(tile, kt); }
  __device__ __forceinline__ void issue(char* tile, int kt) const {
    const int w = wave_id();
#pragma unroll
    for (int j = 0; j < LOADS; ++j) gl2lds(p[j] + (size_t)kt * ROWB, tile + (w * LOADS + j) * 1024);
  }
  // 16-byte chunk c of row r of the staged tile
  __device__ __forceinline__ static const char* at(const char* tile, int r, int c) {
    return tile + r * ROWB + ((c ^ swz(r)) << 4);
  }
};

// Accumulator element q of block (i, j) is C[am0 + 32i + (lane & 31)][bn[j] + 8(q/4) + 4(lane/32) + q%4]:
// for a = q/4 a lane holds 4 consecutive columns of one row.
__device__ __forceinline__ int acc_m(int i, int lane) { return 32 * i + (lane & 31); }
__device__ __forceinline__ int acc_n(int a, int lane) { return 8 * a + 4 * (lane >> 5); }

__device__ __forceinline__ uint2 pack4(float a, float b, float c, float d) {
  typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
  const bf16x4 v = {(bf16)a, (bf16)b, (bf16)c, (bf16)d};
  return __builtin_bit_cast(uint2, v);
}
__device__ __forceinline__ void st8(void* p, uint2 v) { *reinterpret_cast<uint2*>(p) = v; }
// ------------------------------------------------------------------------------------------------
// Epilogue staging. After the main loop the LDS ring is free. Each wave stages 32 rows of its
// NJ blocks of 32 columns as fp32 (row stride 32 NJ + 4 floats, so the 32 rows of one write land in
// distinct banks). It then reads them back row-contiguous, so that global loads and stores move
// whole 128- or 256-byte row segments with 16-byte lanes.
template <int NJ>
struct Stage {
  static constexpr int LD = 32 * NJ + 4;       // staged row stride (floats)
  static constexpr int SIZE = 32 * LD;         // floats per wave
};
constexpr int SLD = Stage<4>::LD;
constexpr int SLAB = Stage<4>::SIZE;

template <int NJ = 4>
__device__ __forceinline__ float* wave_slab(char* smem) {
  return reinterpret_cast<float*>(smem) + wave_id() * Stage<NJ>::SIZE;
}

// rows 32i .. 32i+31 of the wave's blocks; staged column 32j + 8a + 4(lane/32) + b holds block j
template <int MI, int NJ>
__device__ __forceinline__ void stage_rows(float* slab, const f32x16 (&acc)[MI][NJ], int i, int lane) {
#pragma unroll
  for (int j = 0; j < NJ; ++j)
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      float4 v = make_float4(acc[i][j][4 * a], acc[i][j][4 * a + 1], acc[i][j][4 * a + 2], acc[i][j][4 * a + 3]);
      *reinterpret_cast<float4*>(slab + (lane & 31) * Stage<NJ>::LD + 32 * j + acc_n(a, lane)) = v;
    }
}

template <int NJ = 4>
__device__ __forceinline__ void read8(const float* slab, int row, int col, float (&v)[8]) {
  const float4 x = *reinterpret_cast<const float4*>(slab + row * Stage<NJ>::LD + col);
  const float4 y = *reinterpret_cast<const float4*>(slab + row * Stage<NJ>::LD + col + 4);
  v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w; v[4] = y.x; v[5] = y.y; v[6] = y.z; v[7] = y.w;
}

__device__ __forceinline__ uint4 pack8(const float (&v)[8]) {
  const bf16x8 b = {(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3], (bf16)v[4], (bf16)v[5], (bf16)v[6], (bf16)v[7]};
  return __builtin_bit_cast(uint4, b);
}
__device__ __forceinline__ void unpack8(uint4 u, float (&v)[8]) {
  const bf16x8 b = __builtin_bit_cast(bf16x8, u);
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = (float)b[e];
}

// Stores the wave's 32 MI x 32 NJ block of C (columns contiguous from its first column) as bf16.
// out_row(m) gives the output row pointer of the wave's row m at its first column, or null to skip
// the row; ncols limits the columns written. A row is read by 4 NJ lanes, 8 columns each.
template <int MI, int NJ, class OutRow>
__device__ __forceinline__ void store_wave_block(char* smem, const f32x16 (&acc)[MI][NJ], int lane, OutRow out_row,
                                               int ncols) {
  constexpr int LPR = 4 * NJ, RPP = 64 / LPR;   // lanes per row, rows per pass
  float* slab = wave_slab<NJ>(smem);
#pragma unroll
  for (int i = 0; i < MI; ++i) {
    stage_rows(slab, acc, i, lane);
#pragma unroll
    for (int s = 0; s < 32 / RPP; ++s) {
      const int rl = lane / LPR + RPP * s, c0 = (lane % LPR) * 8;
      bf16* o = out_row(32 * i + rl);
      if (o && c0 < ncols) {
        float v[8];
        read8<NJ>(slab, rl, c0, v);
        st16_nt(o + c0, pack8(v));
      }
    }
  }
}

// store_wave_block with the rows staged as bf16 (rounded once, as in store_wave_block) in a
// caller-chosen LDS area, RS rows at a time: wave w uses RS (32 NJ + 8) bf16 from area +
// w RS (32 NJ + 8) 2 bytes. Rows whose out_row is null, and columns from ncols on, are skipped; with
// every row and column stored, that is MI * 32 * 4 NJ / 64 stores per lane. The row stride of 4
// banks mod 64 keeps the staging writes (lane l: row l % 32, 4 columns) conflict-free.
template <int MI, int NJ, int RS = 32, class OutRow>
__device__ __forceinline__ void store_wave_block_bf16(char* area, const f32x16 (&acc)[MI][NJ], int lane, OutRow out_row,
                                                      int ncols = 32 * NJ) {
  static_assert(RS == 32 || RS == 16, "staged rows");
  constexpr int LDB = 32 * NJ + 8;               // staged row stride (bf16)
  constexpr int LPR = 4 * NJ, RPP = 64 / LPR;    // lanes per row, rows per pass
  bf16* st = reinterpret_cast<bf16*>(area) + wave_id() * RS * LDB;
#pragma unroll
  for (int i = 0; i < MI; ++i) {
#pragma unroll
    for (int h = 0; h < 32 / RS; ++h) {
      // the lanes holding rows h RS .. h RS + RS - 1 of the block stage them (LDS accesses of one
      // wave run in order, so these writes follow the previous half's reads)
      if (RS == 32 || (lane & 31) / RS == h) {
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
          for (int a = 0; a < 4; ++a)
            st8(st + ((lane & 31) % RS) * LDB + 32 * j + acc_n(a, lane),
                pack4(acc[i][j][4 * a], acc[i][j][4 * a + 1], acc[i][j][4 * a + 2], acc[i][j][4 * a + 3]));
      }
#pragma unroll
      for (int s = 0; s < RS / RPP; ++s) {
        const int rl = lane / LPR + RPP * s, c0 = (lane % LPR) * 8;
        bf16* o = out_row(32 * i + RS * h + rl);
        if (o && c0 < ncols) st16_nt(o + c0, *reinterpret_cast<const uint4*>(st + rl * LDB + c0));
      }
    }
  }
}

// Writes staged columns [0, ncol) of the 32 staged rows to a pair-contiguous transposed copy.
// dst(c) is the copy's row for staged column c, at the pair column of staged row 0 (null: skip).
// Four lanes cover one column, 8 consecutive pair rows each: one 16-byte store, 64 contiguous bytes
// per column, 16 columns per instruction. (One lane per column, with conflict-free LDS reads but 64
// lines per store instruction, made the dgrad of h 9 % slower.) The row stride is 4 banks mod 64,
// so rows 16 apart share banks: lane groups q = 2, 3 (rows 16-31) read their 8 rows starting from
// the fifth, which puts the four groups of a read on bank offsets 0, 32, 16, 48 (no conflicts; the
// in-order form conflicted 2-way on every read).
template <int NJ = 4, class Dst>
__device__ __forceinline__ void store_transposed(const float* slab, int lane, int ncol, Dst dst) {
  static_assert(Stage<NJ>::LD % 64 == 4, "the read order assumes a row stride of 4 banks mod 64");
  const int rot = 4 * ((lane >> 1) & 1);
  for (int cb = 0; cb < ncol; cb += 16) {
    const int c = cb + (lane >> 2), g8 = 8 * (lane & 3);
    bf16* o = dst(c);
    if (o) {
      // r[t] = row g8 + ((t + rot) & 7): two base addresses with constant offsets
      const float* lo = slab + (g8 + rot) * Stage<NJ>::LD + c;
      const float* hi = slab + (g8 + 4 - rot) * Stage<NJ>::LD + c;
      float r[8];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        r[t] = lo[t * Stage<NJ>::LD];
        r[t + 4] = hi[t * Stage<NJ>::LD];
      }
      const uint4 w = pack8(r);   // rotated groups hold rows 4-7 in the low half: swap the halves
      const uint4 out = rot ? make_uint4(w.z, w.w, w.x, w.y) : w;
      st16(o + g8, out);   // 64 bytes per column: ordinary store (non-temporal partial lines are slow)
    }
  }
}

__device__ __forceinline__ void unpack4(uint2 v, float (&f)[4]) {
  typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
  const bf16x4 b = __builtin_bit_cast(bf16x4, v);
  f[0] = (float)b[0]; f[1] = (float)b[1]; f[2] = (float)b[2]; f[3] = (float)b[3];
}

// Writes staged columns [0, ncol) of the 32 staged rows, quantised along the rows (the pairs), to a
// pair-contiguous transposed fp8 copy. dst(c) is the copy's row for staged column c at the pair
// column of staged row 0 (a multiple of 32), null to skip; sdst(c) is its scale byte.
template <int NJ = 4, class Dst, class SDst>
__device__ __forceinline__ void store_transposed_mx(const float* slab, int lane, int ncol, Dst dst, SDst sdst) {
  // one lane per column: the 32 staged rows of the column are one block of 32, so no shuffles for
  // its amax, and the LDS reads are conflict-free (the 64 lanes read 64 consecutive columns of one
  // row). Measured 3-6 % faster on the MX gate/up and dH GEMMs than four lanes per column.
  for (int c = lane; c < ncol; c += 64) {
    float m = 0.f;
#pragma unroll
    for (int r = 0; r < 32; ++r) m = fmaxf(m, fabsf(slab[r * Stage<NJ>::LD + c]));
    const int s = mx_exponent(m);
    const MxScale sc = mx_scale(s);
    unsigned w[8];
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      const float* col = slab + 4 * g * Stage<NJ>::LD + c;
      w[g] = mx_cvt4(col[0], col[Stage<NJ>::LD], col[2 * Stage<NJ>::LD], col[3 * Stage<NJ>::LD], sc);
    }
    uint8_t* o = dst(c);
    if (o) {
      st16(o, make_uint4(w[0], w[1], w[2], w[3]));
      st16(o + 16, make_uint4(w[4], w[5], w[6], w[7]));
      *sdst(c) = (uint8_t)(s + 127);
    }
  }
}

}  // namespace eng
}  // namespace moe
