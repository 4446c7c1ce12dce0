// Device building blocks shared by the MoE kernels (gfx950 / CDNA4): element traits, the LDS
// tile layout, MFMA micro-steps, global->LDS operand loaders and the double-buffered main loop.
//
// GEMM data movement is counted in 16-byte chunks. One K-tile of an operand occupies one
// 128-byte LDS row per M (or N) index: 64 bf16 or 32 fp32 contraction elements, 8 chunks.
// Chunk c of row r is stored at slot c ^ ((r ^ (r >> 3)) & 7), so that
//   * the MFMA fragment reads (16 rows, same chunk) hit 8 distinct 16-byte slots per 8 lanes;
//   * the transposing stores of contraction-axis-contiguous operands (rows 8 apart, same
//     chunk) hit distinct slots too.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;   // 4 wavefronts of 64
constexpr int kRowBytes = 128;  // one K-tile row in LDS

template <class T> struct Elem;
template <> struct Elem<float> {
  static constexpr int VEC = 4;    // elements per 16-byte chunk
  static constexpr int BK = 32;    // contraction elements per K-tile
};
template <> struct Elem<bf16> {
  static constexpr int VEC = 8;
  static constexpr int BK = 64;
};

__device__ __forceinline__ int lds_slot(int row, int c) { return c ^ ((row ^ (row >> 3)) & 7); }
__device__ __forceinline__ int lds_off(int row, int c) { return row * kRowBytes + (lds_slot(row, c) << 4); }

__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ void st16(void* p, uint4 v) { *reinterpret_cast<uint4*>(p) = v; }
// Epilogue outputs are written once and read by a later kernel. Non-temporal stores keep them from
// displacing, in L2, the operand tiles that other workgroups still reuse (measured 2-5 % per GEMM).
// Only where the lanes of one instruction write whole 128-byte lines: non-temporal stores of
// partial lines measured up to 3.4x slower.
__device__ __forceinline__ void st16_nt(void* p, uint4 v) {
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 w = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(w, reinterpret_cast<u32x4*>(p));
}
__device__ __forceinline__ void st8_nt(void* p, uint2 v) {
  typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
  const u32x2 w = {v.x, v.y};
  __builtin_nontemporal_store(w, reinterpret_cast<u32x2*>(p));
}

// 16-byte load of data read once (the combine's per-pair rows): non-temporal, so that it does not
// stay in L2
__device__ __forceinline__ uint4 ld16_nt(const void* p) {
  typedef unsigned u32x4v __attribute__((ext_vector_type(4)));
  const u32x4v v = __builtin_nontemporal_load(reinterpret_cast<const u32x4v*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// ---------------------------------------------------------------------------------------------
// MFMA micro-step on one 16x16 output block. Lane l supplies row (l & 15) of A and column
// (l & 15) of B, and the 16-byte chunk (l >> 4) of the current 4-chunk contraction step. The
// same lane-to-k assignment is used for both operands, so the k order inside a step does not
// change the sum. Accumulator element q of lane l is C[4*(l >> 4) + q][l & 15].
template <class T> __device__ __forceinline__ void mma16(f32x4& acc, const uint4& a, const uint4& b);

template <> __device__ __forceinline__ void mma16<bf16>(f32x4& acc, const uint4& a, const uint4& b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
}

// fp32: a chunk is 4 contraction elements; four 16x16x4 MFMAs consume one each.
template <> __device__ __forceinline__ void mma16<float>(f32x4& acc, const uint4& a, const uint4& b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.x), __uint_as_float(b.x), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.y), __uint_as_float(b.y), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.z), __uint_as_float(b.z), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.w), __uint_as_float(b.w), acc, 0, 0, 0);
}

// One wave's 64x64 sub-tile over one K-tile: A rows arow0 + 16*i, B rows brow[j].
template <class T>
__device__ __forceinline__ void wave_mma(f32x4 (&acc)[4][4], const char* ldsA, const char* ldsB,
                                         int arow0, const int (&brow)[4], int lane) {
  const int lr = lane & 15, lg = lane >> 4;
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    uint4 fa[4], fb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) fa[i] = ld16(ldsA + lds_off(arow0 + 16 * i + lr, 4 * s + lg));
#pragma unroll
    for (int j = 0; j < 4; ++j) fb[j] = ld16(ldsB + lds_off(brow[j] + lr, 4 * s + lg));
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) mma16<T>(acc[i][j], fa[i], fb[j]);
  }
}

// ---------------------------------------------------------------------------------------------
// Operand loaders. Each moves one K-tile (128 bytes of contraction per row) of a ROWS-row operand
// tile from global memory into registers (fetch), then into the LDS layout above (store).

// K-major operand: row i is contiguous along K. This thread moves chunk (tid & 7) of rows
// (tid >> 3) + 32*i. p[i] points at that chunk of K-tile 0, or is null for a zero row.
template <int ROWS>
struct KLoader {
  static constexpr int N = ROWS / 32;
  const char* p[N];
  uint4 r[N];
  __device__ __forceinline__ void fetch(int kt) {
#pragma unroll
    for (int i = 0; i < N; ++i)
      r[i] = p[i] ? ld16(p[i] + (size_t)kt * kRowBytes) : make_uint4(0, 0, 0, 0);
  }
  __device__ __forceinline__ void store(char* lds, int tid) const {
#pragma unroll
    for (int i = 0; i < N; ++i) st16(lds + lds_off((tid >> 3) + 32 * i, tid & 7), r[i]);
  }
};

// MN-major operand: each contraction index k owns a contiguous row of ROWS elements (the tile's
// M or N extent). A micro-block is 4 consecutive k by one 16-byte chunk of the row. It is loaded
// as 4 chunks, transposed in registers, and stored as VEC LDS rows of 4 contraction elements.
// Src::row(k) returns the byte address of element 0 of contraction row k of this tile, or null
// when k is out of range (that row reads as zero).
template <class T, int ROWS, class Src>
struct MNLoader {
  static constexpr int VEC = Elem<T>::VEC;
  static constexpr int BK = Elem<T>::BK;
  static constexpr int NCOL = ROWS / VEC;      // 16-byte chunks per contraction row
  static constexpr int NMB = 2 * ROWS / kThreads;  // micro-blocks per thread ((BK/4)*NCOL == 2*ROWS)
  Src src;
  int kq[NMB], mc[NMB];
  uint4 r[NMB][4];
  __device__ __forceinline__ void init(int tid) {
#pragma unroll
    for (int i = 0; i < NMB; ++i) {
      const int mb = tid + kThreads * i;
      kq[i] = mb / NCOL;
      mc[i] = mb % NCOL;
    }
  }
  __device__ __forceinline__ void fetch(int kt) {
#pragma unroll
    for (int i = 0; i < NMB; ++i)
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const char* p = src.row(kt * BK + 4 * kq[i] + kk);
        r[i][kk] = p ? ld16(p + 16 * mc[i]) : make_uint4(0, 0, 0, 0);
      }
  }
  __device__ __forceinline__ void store(char* lds, int) const;
};

template <class T, int ROWS, class Src>
__device__ __forceinline__ void MNLoader<T, ROWS, Src>::store(char* lds, int) const {
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int i = 0; i < NMB; ++i) {
      const uint32_t* w0 = reinterpret_cast<const uint32_t*>(&r[i][0]);
      const uint32_t* w1 = reinterpret_cast<const uint32_t*>(&r[i][1]);
      const uint32_t* w2 = reinterpret_cast<const uint32_t*>(&r[i][2]);
      const uint32_t* w3 = reinterpret_cast<const uint32_t*>(&r[i][3]);
      const int c = kq[i] >> 1, half = (kq[i] & 1) * 8;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int sh = (j & 1) * 16;
        const uint32_t e0 = (w0[j >> 1] >> sh) & 0xFFFFu, e1 = (w1[j >> 1] >> sh) & 0xFFFFu;
        const uint32_t e2 = (w2[j >> 1] >> sh) & 0xFFFFu, e3 = (w3[j >> 1] >> sh) & 0xFFFFu;
        const int row = mc[i] * 8 + j;
        uint2 v = make_uint2(e0 | (e1 << 16), e2 | (e3 << 16));
        *reinterpret_cast<uint2*>(lds + lds_off(row, c) + half) = v;
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < NMB; ++i) {
      const uint32_t* w0 = reinterpret_cast<const uint32_t*>(&r[i][0]);
      const uint32_t* w1 = reinterpret_cast<const uint32_t*>(&r[i][1]);
      const uint32_t* w2 = reinterpret_cast<const uint32_t*>(&r[i][2]);
      const uint32_t* w3 = reinterpret_cast<const uint32_t*>(&r[i][3]);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int row = mc[i] * 4 + j;
        st16(lds + lds_off(row, kq[i]), make_uint4(w0[j], w1[j], w2[j], w3[j]));
      }
    }
  }
}

// ---------------------------------------------------------------------------------------------
// Double-buffered main loop over nk K-tiles for a 128x128 block tile computed by 4 waves, each
// a 64x64 sub-tile (A rows arow0.., B rows brow[]). smem holds 2 x (A 16 KB + B 16 KB).
// Global loads for K-tile kt+1 are in flight while the MFMAs of K-tile kt run.
constexpr int kTileBytes = 128 * kRowBytes;     // 16 KB per operand per buffer
constexpr int kSmemBytes = 4 * kTileBytes;      // 64 KB

template <class T, class LA, class LB>
__device__ __forceinline__ void mainloop(f32x4 (&acc)[4][4], char* smem, LA& la, LB& lb, int nk,
                                         int arow0, const int (&brow)[4]) {
  const int tid = threadIdx.x, lane = tid & 63;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (nk <= 0) return;
  la.fetch(0);
  lb.fetch(0);
  la.store(smem, tid);
  lb.store(smem + kTileBytes, tid);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    char* cur = smem + (kt & 1) * 2 * kTileBytes;
    char* nxt = smem + ((kt + 1) & 1) * 2 * kTileBytes;
    const bool more = kt + 1 < nk;
    if (more) {
      la.fetch(kt + 1);
      lb.fetch(kt + 1);
    }
    wave_mma<T>(acc, cur, cur + kTileBytes, arow0, brow, lane);
    if (more) {
      la.store(nxt, tid);
      lb.store(nxt + kTileBytes, tid);
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------------------------
// Work distribution. Workgroups are dispatched to the 8 XCDs round-robin by workgroup id, and
// each XCD has its own L2. Persistent kernels therefore give each XCD one contiguous range of
// the tile list (tiles of the same expert share operands). The grid must be a multiple of 8.
struct XcdRange {
  int begin, end, stride, first;
};
__device__ __forceinline__ XcdRange xcd_range(int total) {
  const int per_xcd_blocks = gridDim.x >> 3;
  const int xcd = blockIdx.x & 7;
  const int per = (total + 7) >> 3;
  XcdRange r;
  r.begin = xcd * per;
  r.end = min(total, r.begin + per);
  r.stride = per_xcd_blocks;
  r.first = r.begin + (blockIdx.x >> 3);
  return r;
}

// Non-persistent grids: logical block id such that consecutive logical ids share an XCD.
__device__ __forceinline__ int xcd_logical_block(int nblocks) {
  const int b = blockIdx.x;
  const int q = nblocks >> 3, rem = nblocks & 7, x = b & 7;
  const int base = x < rem ? x * (q + 1) : rem * (q + 1) + (x - rem) * q;
  return base + (b >> 3);
}

template <class T> __device__ __forceinline__ T cvt_out(float v) { return (T)v; }

// The combines (forward y, backward dx): a wavefront sums one part of a row (128 chunks of 16 bytes:
// 2048 bf16) for tpw consecutive tokens, loading all their pair positions with one instruction (lane
// q holds slot q % k of token q / k), then gathering token after token. Where few of a token's slots
// are local (an expert share of at most a quarter of the experts), several tokens per wavefront
// spend one pair-position round trip on several short gathers (forward combine 8 %, backward 18 %
// faster on a 16-of-128 share); with every slot local, the gathers are long and one token per
// wavefront keeps more of them in flight (4 tokens: 4-7 % slower).
__host__ __device__ constexpr int combine_tpw(int k, int E_local, int E_total) {
  return 4 * E_local > E_total ? 1 : (64 / k < 4 ? 64 / k : 4);
}

// dst row part `part` (of nparts) = the sum, in slot order and fp32, of the source rows src[pp] of the
// k slots whose pair positions pp sit in lanes slot0 .. slot0+k-1 of ppv (pp < 0: not local). Each
// lane takes two chunks, so 16 slot rows are in flight per lane. The loop is uniform over the wave,
// with every lane active at the readlane (a value computed under a narrower exec mask is undefined in
// the lanes outside it, and the slots' lanes can lie past a short row's last chunk): lanes past the
// row's end load zeros and store nothing.
template <class T, int VEC>
__device__ __forceinline__ void combine_row_part(const T* __restrict__ src, int ppv, int slot0, int k, int H, int nch,
                                                 int part, int nparts, int lane, T* __restrict__ dst) {
  for (int cb = 128 * part; cb < nch; cb += 128 * nparts) {
    const int c0 = cb + lane;
    float acc[2][VEC];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int v = 0; v < VEC; ++v) acc[h][v] = 0.f;
    for (int j0 = 0; j0 < k; j0 += 8) {
      uint4 raw[2][8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int ps = j0 + u < k ? __builtin_amdgcn_readlane(ppv, slot0 + j0 + u) : -1;
#pragma unroll
        for (int h = 0; h < 2; ++h)
          raw[h][u] = ps >= 0 && c0 + 64 * h < nch ? ld16_nt(src + (size_t)ps * H + (size_t)(c0 + 64 * h) * VEC)
                                                   : make_uint4(0u, 0u, 0u, 0u);
      }
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const T* ev = reinterpret_cast<const T*>(&raw[h][u]);
#pragma unroll
          for (int v = 0; v < VEC; ++v) acc[h][v] += (float)ev[v];
        }
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      uint4 res;
      T* r = reinterpret_cast<T*>(&res);
#pragma unroll
      for (int v = 0; v < VEC; ++v) r[v] = cvt_out<T>(acc[h][v]);
      if (c0 + 64 * h < nch) st16(dst + (size_t)(c0 + 64 * h) * VEC, res);
    }
  }
}

// Cross-lane moves inside a 16-lane row through DPP (a VALU source modifier: no LDS round trip, unlike
// __shfl, which compiles to ds_bpermute_b32). Every lane of the row must be active.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xf, 0xf, false));
}
template <int CTRL>
__device__ __forceinline__ unsigned dpp_mov(unsigned v) {
  return (unsigned)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xf, 0xf, false);
}
constexpr int kDppXor1 = 0xb1;         // quad_perm [1,0,3,2]: the lane's xor-1 partner
constexpr int kDppXor2 = 0x4e;         // quad_perm [2,3,0,1]: xor 2
constexpr int kDppHalfMirror = 0x141;  // row_half_mirror: lane i of each 8 takes lane 7 - i
constexpr int kDppMirror = 0x140;      // row_mirror: lane i of each 16 takes lane 15 - i
// Sum over aligned groups of 8 (16) lanes, every lane getting the group's sum. The last step takes
// the mirrored lane instead of the xor-4 (xor-8) one: after the quad steps all lanes of a quad hold
// the same bits, so the additions are the ones of a xor butterfly, bit for bit.
__device__ __forceinline__ float group_sum8(float v) {
  v += dpp_mov<kDppXor1>(v);
  v += dpp_mov<kDppXor2>(v);
  return v + dpp_mov<kDppHalfMirror>(v);
}
__device__ __forceinline__ float group_sum16(float v) {
  v = group_sum8(v);
  return v + dpp_mov<kDppMirror>(v);
}
__device__ __forceinline__ float quad_max(float m) {
  m = fmaxf(m, dpp_mov<kDppXor1>(m));
  return fmaxf(m, dpp_mov<kDppXor2>(m));
}
__device__ __forceinline__ float group_max8(float m) {
  m = quad_max(m);
  return fmaxf(m, dpp_mov<kDppHalfMirror>(m));
}

// sigma(z) = 1 / (1 + e^-z), with the hardware reciprocal (v_rcp_f32, about 1 ulp) instead of an
// IEEE division: the division's scale/Newton/fixup sequence was about ten instructions per element
// in the SwiGLU and dSwiGLU epilogues, whose VALU work the matrix cores wait on. For large -z the
// exponential overflows to +inf and the reciprocal gives 0, as the division does.
__device__ __forceinline__ float sigmoidf_(float z) { return __builtin_amdgcn_rcpf(1.0f + __expf(-z)); }

}  // namespace moe
