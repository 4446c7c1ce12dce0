// MXFP8 grouped-GEMM engine for gfx950 and the six expert GEMMs of the fused MoE layer in the MX
// precision modes ("Supporto di precisione e vincoli hardware" on "Prime Mega MoE: il kernel che
// accelera il training AI del 55%" names MXFP8 among the kernel's modes; the layer itself is the
// one of "A Magia da Fusão" on "IA: MoE Kernel 3x Mais Rápido Chegou!").
//
// Engine:
//  * v_mfma_scale_f32_32x32x64_f8f6f4 with E4M3 operands. Lane l holds row l%32 of an operand:
//    bytes 0-15 are contraction elements 16(l/32) + 0..15 and bytes 16-31 are elements
//    32 + 16(l/32) + 0..15. The block scale of (row i, 32-element block b) comes from lane i + 32b.
//  * A K-tile is 128 fp8 elements = 128 bytes per row (whole cache lines, as in the bf16 engine),
//    two 64-deep MFMA steps. The data tiles, the swizzle and the K-major loader are the bf16
//    engine's (engine.h); step s reads chunks 4s + l/32 and 4s + 2 + l/32 of each row. The ring
//    has 2 stages of 66 KB.
//  * Every operand is K-major. The quantise kernels and the GEMM epilogues write them that way,
//    with scales in [rows][K/32] byte arrays, except the pair-contiguous copies (K = the pairs),
//    whose scales are K-tile-major, [Q/128][rows][4] (tscale_at). Either way a K-tile's 4 scale
//    bytes of a row are one dword, kstride bytes after the previous K-tile's (4, or 4 rows; scale
//    bases and row lengths are multiples of 4 bytes: rows of H/32, F/32 or 2F/32 bytes, expert
//    segments padded to 128 pairs). Per stage, each thread moves one
//    scale dword per operand into LDS (global_load_lds_dword). Dword d of the stage's scale area
//    holds the row of quadrant half d/128, 32-row block d%4 and row (d%128)/4 of that block. A lane
//    reads the scales of its four 32-row blocks with one 16-byte LDS read, and takes byte
//    2s + l/32 in step s.
//  * Main loop per K-tile: step 0's MFMAs of row blocks 0-1, the reads of step 1's fragments, step
//    0's MFMAs of row blocks 2-3 and step 1's of blocks 0-1; then wait + barrier, the issue of
//    K-tile kt+2, the reads of the next K-tile's step-0 fragments, and step 1's MFMAs of blocks
//    2-3. Fragments are double-buffered, so LDS reads overlap MFMAs.
//  * Epilogues quantise in registers where the next GEMM needs an fp8 operand. 4 lanes hold a
//    block of 32 along F (row pass) or along the pairs (transposed pass); two shuffles give its
//    amax.
#include <type_traits>

#include "engine.h"
#include "moe_internal.h"
#include "mx_device.h"

namespace moe {
namespace {

using namespace eng;

typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int KTILE = 128;                     // fp8 contraction elements per K-tile
typedef KRows<128> KOp;                        // 128 bytes per row per K-tile
constexpr int LOADS = KOp::LOADS;              // 8 direct-to-LDS loads per lane per operand per K-tile
constexpr int STAGES = 2;                      // LDS ring depth (2 x 66 KB)
constexpr int OPB = 32768;                     // data bytes per operand per stage (256 rows x 128 B)
constexpr int STB = 2 * OPB;
constexpr int SCB = 1024;                      // scale bytes per operand per stage (256 dwords)
constexpr int STB_MX = STB + 2 * SCB;          // stage: A data, B data, A scales, B scales
constexpr int VM_PER_TILE = 2 * LOADS + 2;     // direct-to-LDS loads per lane per K-tile
constexpr int SMEM_MX = STAGES * STB_MX > 8 * SLAB * 4 ? STAGES * STB_MX : 8 * SLAB * 4;
#define MX_SMEM __shared__ __attribute__((aligned(1024))) char smem[SMEM_MX];

// lane i copies 4 bytes from g into lds + 4*i (lds wave-uniform); see gl2lds
__device__ __forceinline__ void gl2lds_dword(const void* g, char* lds) {
  const unsigned off = __builtin_amdgcn_readfirstlane((unsigned)(uintptr_t)lds);   // the LDS address
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, off" ::"s"(off), "v"(g) : "memory", "m0");
}

// The operand-tile row whose scale dword this thread moves: quadrant half h, block j, row l32.
__device__ __forceinline__ int sc_half() { return threadIdx.x >> 7; }
__device__ __forceinline__ int sc_blk() { return threadIdx.x & 3; }
__device__ __forceinline__ int sc_row32() { return (threadIdx.x & 127) >> 2; }

// scale row of this thread, and the scale column of K-tile 0 (a multiple of 4)
struct SOp {
  const uint8_t* row;
  int cbase;
  int kstride = 4;   // bytes from one K-tile's scale dword to the next: 4 in [rows][K/32] arrays
  __device__ __forceinline__ void issue(char* area, int kt) const {
    gl2lds_dword(row + cbase + (size_t)kstride * kt, area + wave_id() * 256);
  }
};

__device__ __forceinline__ i32x8 frag8(const char* tile, int row0, int s, int lane) {
  const int r = row0 + (lane & 31), h = lane >> 5;
  const uint4 lo = *reinterpret_cast<const uint4*>(KOp::at(tile, r, 4 * s + h));
  const uint4 hi = *reinterpret_cast<const uint4*>(KOp::at(tile, r, 4 * s + 2 + h));
  const i32x8 v = {(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
  return v;
}

struct Frags {
  i32x8 a[4], b[4];
  uint4 sa, sb;   // scale dwords of the lane's four A blocks and four B blocks
};

// step s of the K-tile staged at st
__device__ __forceinline__ void read_frags_mx(Frags& f, const char* st, int s, int am0, const int (&bn)[4], int wm,
                                              int wn, int lane) {
#pragma unroll
  for (int i = 0; i < 4; ++i) f.a[i] = frag8(st, am0 + 32 * i, s, lane);
#pragma unroll
  for (int j = 0; j < 4; ++j) f.b[j] = frag8(st + OPB, bn[j], s, lane);
  f.sa = *reinterpret_cast<const uint4*>(st + 2 * OPB + (wm * 128 + (lane & 31) * 4) * 4);
  f.sb = *reinterpret_cast<const uint4*>(st + 2 * OPB + SCB + (wn * 128 + (lane & 31) * 4) * 4);
}

// MFMAs of row blocks i0, i0+1 (B fragment first: each accumulator block holds the transposed
// 32x32 block, as in the bf16 engine). Each MFMA is followed in issue order by RPM of the LDS
// fragment reads around it, so that one wave per SIMD keeps its matrix core fed while it reads.
template <int RPM = 1>
__device__ __forceinline__ void mma_half(f32x16 (&acc)[4][4], const Frags& f, int i0, int sela, int selb) {
  const unsigned sa[4] = {f.sa.x, f.sa.y, f.sa.z, f.sa.w};
  const unsigned sb[4] = {f.sb.x, f.sb.y, f.sb.z, f.sb.w};
#pragma unroll
  for (int ii = 0; ii < 2; ++ii) {
    const int i = i0 + ii;
    const int as = (int)((sa[i] >> sela) & 0xffu);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int bs = (int)((sb[j] >> selb) & 0xffu);
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(f.b[j], f.a[i], acc[i][j], 0, 0, 0, bs, 0, as);
    }
  }
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, RPM, 0);
  }
}

__device__ __forceinline__ void wait_tile_mx(int younger) {
  if (younger >= 3) wait_vm<3 * VM_PER_TILE>();
  else if (younger == 2) wait_vm<2 * VM_PER_TILE>();
  else if (younger == 1) wait_vm<VM_PER_TILE>();
  else wait_vm<0>();
}

template <class LA, class LB>
__device__ __forceinline__ void issue_tile(char* st, const LA& la, const LB& lb, const SOp& sa, const SOp& sb, int kt) {
  la.issue(st, kt);
  lb.issue(st + OPB, kt);
  sa.issue(st + 2 * OPB, kt);
  sb.issue(st + 2 * OPB + SCB, kt);
}

// One K-tile (see the engine notes above). The wait, barrier and fragment reads run unconditionally:
// past the last K-tile they reread a stage that is no longer refilled, and the fragments go unused.
// Keeping them unconditional lets the compiler hold both fragment sets in registers.
template <class LA, class LB>
__device__ __forceinline__ void ktile_mx(f32x16 (&acc)[4][4], char* smem, const LA& la, const LB& lb, const SOp& sa,
                                         const SOp& sb, int kt, int nk, Frags& f0, Frags& f1, int am0,
                                         const int (&bn)[4], int wm, int wn, int lane) {
  char* cur = smem + (kt % STAGES) * STB_MX;
  const int h8 = 8 * (lane >> 5);
  mma_half(acc, f0, 0, h8, h8);
  read_frags_mx(f1, cur, 1, am0, bn, wm, wn, lane);
  mma_half(acc, f0, 2, h8, h8);
  mma_half(acc, f1, 0, 16 + h8, 16 + h8);
  wait_tile_mx(min(nk - 2 - kt, STAGES - 2));
  block_sync();
  if (kt + STAGES < nk) issue_tile(cur, la, lb, sa, sb, kt + STAGES);
  read_frags_mx(f0, smem + ((kt + 1) % STAGES) * STB_MX, 0, am0, bn, wm, wn, lane);
  mma_half<2>(acc, f1, 2, 16 + h8, 16 + h8);
}

// nk K-tiles of 128 elements (every scale base a multiple of 4 scale columns).
template <class LA, class LB>
__device__ __forceinline__ void mainloop_mx(f32x16 (&acc)[4][4], char* smem, const LA& la, const LB& lb, const SOp& sa,
                                            const SOp& sb, int nk, int am0, const int (&bn)[4], int wm, int wn) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;
  if (nk <= 0) return;
  wait_vm<0>();   // stores of the previous tile's epilogue must not count against the ring below
  block_sync();   // and every wave is done reading its epilogue staging slab
#pragma unroll
  for (int s = 0; s < STAGES; ++s)
    if (s < nk) issue_tile(smem + s * STB_MX, la, lb, sa, sb, s);
  wait_tile_mx(min(nk - 1, STAGES - 1));
  block_sync();
  Frags f0, f1;
  read_frags_mx(f0, smem, 0, am0, bn, wm, wn, lane);
  for (int kt = 0; kt < nk; ++kt) ktile_mx(acc, smem, la, lb, sa, sb, kt, nk, f0, f1, am0, bn, wm, wn, lane);
  block_sync();
}

// Blockwise FP8 form of store_transposed_mx: the staged column c (one lane per column) is written
// with the exponent sx(c) of its whole block of pairs, found beforehand.
template <class Dst, class SDst, class Sx>
__device__ __forceinline__ void store_transposed_fixed(const float* slab, int lane, int ncol, Dst dst, SDst sdst,
                                                       Sx sx) {
  for (int c = lane; c < ncol; c += 64) {
    const int s = sx(c);
    const MxScale sc = mx_scale(s);
    unsigned w[8];
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      const float* col = slab + 4 * g * SLD + c;
      w[g] = mx_cvt4(col[0], col[SLD], col[2 * SLD], col[3 * SLD], sc);
    }
    uint8_t* o = dst(c);
    if (o) {
      st16(o, make_uint4(w[0], w[1], w[2], w[3]));
      st16(o + 16, make_uint4(w[4], w[5], w[6], w[7]));
      *sdst(c) = (uint8_t)(s + 127);
    }
  }
}

// largest magnitude of staged column c over the 32 staged rows (8 reads in flight at a time: fully
// unrolled, the compiler issued all of them at once and spilled the values)
__device__ __forceinline__ float column_amax(const float* slab, int c) {
  float m = 0.f;
#pragma unroll 8
  for (int r = 0; r < 32; ++r) m = fmaxf(m, fabsf(slab[r * SLD + c]));
  return m;
}

// ------------------------------------------------------------------------------------------------
// forward: [a | b] = gather(x) [W_gate; W_up]^T; epilogue writes ab (bf16), hw = w silu(a) b as fp8
// along F (the down GEMM's A operand) and as fp8 along the pairs (the down weight gradient's B).
// Each output may be null, and is then not written (activation checkpointing: the forward writes
// the fp8 hw along F alone, the backward's recompute ab and the copy along the pairs).
// Blockwise FP8 epilogue of the gate/up GEMM. w h is quantised along F in blocks of 128 columns,
// which the two waves wn = 0, 1 of a row share (64 columns each), and along the pairs in blocks of
// the wave's 128 rows. Pass 1 computes h, writes a and b, each row's maximum over the wave's 64
// columns (into LDS past the four staging slabs, for the partner wave) and each column's maximum
// over the 128 rows. After a barrier, pass 2 recomputes h (the same operations on the same values)
// and writes both fp8 copies with those scales.
__device__ __forceinline__ void epilogue_gateup_blk(const FwdParams& p, const f32x16 (&acc)[4][4], char* smem,
                                                    float* slab, const float (&wrow)[4], int lane, int w, int wm,
                                                    int r0, int seg_end, int f0, int qend, int colq) {
  bf16* __restrict__ ab = static_cast<bf16*>(p.ab);
  const int F = p.F;
  float* rmax = reinterpret_cast<float*>(smem) + 4 * SLAB;   // [4 waves][128 rows]
  auto hrow = [&](int i, int s, float (&hv)[8], bool write_ab) {
    const int rl = (lane >> 3) + 8 * s, c0 = (lane & 7) * 8;
    const float wt = __shfl(wrow[i], rl);
    const int r = r0 + 128 * wm + 32 * i + rl;
    if (r < seg_end) {
      float av[8], bv[8];
      read8(slab, rl, c0, av);
      read8(slab, rl, 64 + c0, bv);
#pragma unroll
      for (int e = 0; e < 8; ++e) hv[e] = wt * (av[e] * sigmoidf_(av[e]) * bv[e]);
      if (write_ab && ab) {
        bf16* abr = ab + (size_t)r * 2 * F + f0 + c0;
        st16_nt(abr, pack8(av));
        st16_nt(abr + F, pack8(bv));
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) hv[e] = 0.f;
    }
  };
  auto put_slab = [&](int s, const float (&hv)[8]) {
    const int rl = (lane >> 3) + 8 * s, c0 = (lane & 7) * 8;
    *reinterpret_cast<float4*>(slab + rl * SLD + c0) = make_float4(hv[0], hv[1], hv[2], hv[3]);
    *reinterpret_cast<float4*>(slab + rl * SLD + c0 + 4) = make_float4(hv[4], hv[5], hv[6], hv[7]);
  };
  float cmax = 0.f;   // column `lane` of the wave's 64, over its 128 rows
  auto pass1 = [&](auto I) {
    constexpr int i = decltype(I)::value;
    stage_rows(slab, acc, i, lane);
#pragma unroll 1
    for (int s = 0; s < 4; ++s) {
      float hv[8];
      hrow(i, s, hv, true);
      float m = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf(hv[e]));
      m = group_max8(m);
      if ((lane & 7) == 0) rmax[w * 128 + 32 * i + (lane >> 3) + 8 * s] = m;
      put_slab(s, hv);
    }
    cmax = fmaxf(cmax, column_amax(slab, lane));
  };
  pass1(std::integral_constant<int, 0>{});
  pass1(std::integral_constant<int, 1>{});
  pass1(std::integral_constant<int, 2>{});
  pass1(std::integral_constant<int, 3>{});
  block_sync();   // the partner wave's row maxima
  const int scol = fp8b_exponent(cmax);
  auto pass2 = [&](auto I) {
    constexpr int i = decltype(I)::value;
    stage_rows(slab, acc, i, lane);
#pragma unroll 1
    for (int s = 0; s < 4; ++s) {
      float hv[8];
      hrow(i, s, hv, false);
      const int rl = (lane >> 3) + 8 * s, c0 = (lane & 7) * 8;
      const int r = r0 + 128 * wm + 32 * i + rl;
      const int sx = fp8b_exponent(fmaxf(rmax[w * 128 + 32 * i + rl], rmax[(w ^ 1) * 128 + 32 * i + rl]));
      if (r < seg_end && p.hwq) {
        *reinterpret_cast<uint2*>(p.hwq + (size_t)r * F + f0 + c0) = mx_encode8(hv, sx);
        if ((lane & 3) == 0) p.hws[(size_t)r * (F / 32) + (f0 + c0) / 32] = (uint8_t)(sx + 127);
      }
      put_slab(s, hv);
    }
    const int colb = colq + 32 * i;
    if (p.hwtq)
      store_transposed_fixed(
        slab, lane, 64, [&](int c) { return colb < qend ? p.hwtq + (size_t)(f0 + c) * p.qc + colb : nullptr; },
        [&](int c) { return p.hwts + tscale_at(F, f0 + c, colb); }, [&](int) { return scol; });
  };
  pass2(std::integral_constant<int, 0>{});
  pass2(std::integral_constant<int, 1>{});
  pass2(std::integral_constant<int, 2>{});
  pass2(std::integral_constant<int, 3>{});
}

template <bool BLK>
__global__ __launch_bounds__(NTHR, 1) void k_gateup_mx(FwdParams p) {
  MX_SMEM
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, wm = w >> 1, wn = w & 1;
  bf16* __restrict__ ab = static_cast<bf16*>(p.ab);
  const int H = p.H, F = p.F, ntn = F / 128, hs = H / 32;
  const XcdRange xr = xcd_range(*p.num_mtiles2 * ntn);
  const int bn[4] = {64 * wn, 64 * wn + 32, 128 + 64 * wn, 128 + 64 * wn + 32};
  const int arow_s = 128 * sc_half() + 32 * sc_blk() + sc_row32();
  const int brow_s = 128 * (sc_blk() >> 1) + 64 * sc_half() + 32 * (sc_blk() & 1) + sc_row32();
  for (int tile = xr.first; tile < xr.end; tile += xr.stride) {
    const int mt = tile / ntn, nt = tile - mt * ntn;
    const int2 me = p.mtile2[mt];
    const int e = me.x, r0 = me.y, seg_end = p.offsets[e + 1];
    KOp la, lb;
#pragma unroll
    for (int j = 0; j < LOADS; ++j) {
      const int row = KOp::row_of(j), c = KOp::chunk_of(j);
      const int r = min(r0 + row, seg_end - 1);
      la.p[j] = reinterpret_cast<const char*>(p.xq + (size_t)p.ptok[r] * H) + 16 * c;
      const uint8_t* wrow = row < 128 ? p.wgq + ((size_t)e * F + nt * 128 + row) * H
                                      : p.wuq + ((size_t)e * F + nt * 128 + row - 128) * H;
      lb.p[j] = reinterpret_cast<const char*>(wrow) + 16 * c;
    }
    const SOp sa{p.xs + (size_t)p.ptok[min(r0 + arow_s, seg_end - 1)] * hs, 0};
    const SOp sb{brow_s < 128 ? p.wgs + ((size_t)e * F + nt * 128 + brow_s) * hs
                              : p.wus + ((size_t)e * F + nt * 128 + brow_s - 128) * hs, 0};
    int prow[4];   // slots of the wave's rows; their routing weights are loaded after the main loop
#pragma unroll
    for (int i = 0; i < 4; ++i) prow[i] = p.perm[min(r0 + 128 * wm + acc_m(i, lane), seg_end - 1)];
    f32x16 acc[4][4];
    mainloop_mx(acc, smem, la, lb, sa, sb, H / KTILE, 128 * wm, bn, wm, wn);
    float wrow[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) wrow[i] = p.weight[prow[i]];
    float* slab = wave_slab(smem);
    const int f0 = nt * 128 + 64 * wn;
    const int qend = p.qoff[e + 1];
    const int colq = p.qoff[e] + (r0 - p.offsets[e]) + 128 * wm;
    if constexpr (BLK) {
      epilogue_gateup_blk(p, acc, smem, slab, wrow, lane, w, wm, r0, seg_end, f0, qend, colq);
      continue;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      stage_rows(slab, acc, i, lane);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int rl = (lane >> 3) + 8 * s, c0 = (lane & 7) * 8;
        const float wt = __shfl(wrow[i], rl);
        const int r = r0 + 128 * wm + 32 * i + rl;
        const bool ok = r < seg_end;
        float hv[8];
        if (ok) {
          float av[8], bv[8];
          read8(slab, rl, c0, av);
          read8(slab, rl, 64 + c0, bv);
#pragma unroll
          for (int e = 0; e < 8; ++e) hv[e] = wt * (av[e] * sigmoidf_(av[e]) * bv[e]);
          if (ab) {
            bf16* abr = ab + (size_t)r * 2 * F + f0 + c0;
            st16_nt(abr, pack8(av));
            st16_nt(abr + F, pack8(bv));
          }
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) hv[e] = 0.f;
        }
        const int sx = mx_exponent(mx_amax_x4(hv));
        if (ok && p.hwq) {
          *reinterpret_cast<uint2*>(p.hwq + (size_t)r * F + f0 + c0) = mx_encode8(hv, sx);
          if ((lane & 3) == 0) p.hws[(size_t)r * (F / 32) + (f0 + c0) / 32] = (uint8_t)(sx + 127);
        }
        *reinterpret_cast<float4*>(slab + rl * SLD + c0) = make_float4(hv[0], hv[1], hv[2], hv[3]);
        *reinterpret_cast<float4*>(slab + rl * SLD + c0 + 4) = make_float4(hv[4], hv[5], hv[6], hv[7]);
      }
      const int colb = colq + 32 * i;
      if (p.hwtq)
        store_transposed_mx(
            slab, lane, 64, [&](int c) { return colb < qend ? p.hwtq + (size_t)(f0 + c) * p.qc + colb : nullptr; },
            [&](int c) { return p.hwts + tscale_at(F, f0 + c, colb); });
    }
  }
}

// forward: o' = hw W_down[e]^T (contraction over F)
__global__ __launch_bounds__(NTHR, 1) void k_down_mx(FwdParams p) {
  MX_SMEM
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, wm = w >> 1, wn = w & 1;
  bf16* __restrict__ o = static_cast<bf16*>(p.o);
  const int H = p.H, F = p.F, ntn = H / TILE, fs = F / 32;
  const XcdRange xr = xcd_range(*p.num_mtiles2 * ntn);
  const int bn[4] = {128 * wn, 128 * wn + 32, 128 * wn + 64, 128 * wn + 96};
  const int row_s = 128 * sc_half() + 32 * sc_blk() + sc_row32();
  for (int tile = xr.first; tile < xr.end; tile += xr.stride) {
    const int mt = tile / ntn, nt = tile - mt * ntn;
    const int2 me = p.mtile2[mt];
    const int e = me.x, r0 = me.y, seg_end = p.offsets[e + 1];
    KOp la, lb;
#pragma unroll
    for (int j = 0; j < LOADS; ++j) {
      const int row = KOp::row_of(j), c = KOp::chunk_of(j);
      const int r = min(r0 + row, seg_end - 1);
      la.p[j] = reinterpret_cast<const char*>(p.hwq + (size_t)r * F) + 16 * c;
      lb.p[j] = reinterpret_cast<const char*>(p.wdq + ((size_t)e * H + nt * TILE + row) * F) + 16 * c;
    }
    const SOp sa{p.hws + (size_t)min(r0 + row_s, seg_end - 1) * fs, 0};
    const SOp sb{p.wds + ((size_t)e * H + nt * TILE + row_s) * fs, 0};
    f32x16 acc[4][4];
    mainloop_mx(acc, smem, la, lb, sa, sb, F / KTILE, 128 * wm, bn, wm, wn);
    const int rq = r0 + 128 * wm;
    bf16* const oq = o + nt * TILE + 128 * wn;
    store_wave_block(smem, acc, lane, [&](int m) { return rq + m < seg_end ? oq + (size_t)(rq + m) * H : nullptr; }, 128);
  }
}

// backward: u = gather(dY) W_down[e] (contraction over H, B = W_down[e]^T quantised along H);
// epilogue writes g partials, and da, db as fp8 along F (dgrad A) and along the pairs (wgrad A)
// Blockwise FP8 epilogue of the dH GEMM. A row's 128 columns of da (and of db) in this wave are one
// block along F (16 lanes: four shuffles give its amax), so the row copies are written in pass 1
// together with the g partials. Along the pairs, a column's block is the wave's 128 rows: pass 1 also
// takes each column's maximum, and pass 2 recomputes da and db (the same operations on the same
// values) and writes the transposed copies with those scales.
__device__ __forceinline__ void epilogue_dh_blk(const BwdParams& p, const f32x16 (&acc)[4][4], float* slab,
                                                float* slab2, const float (&wrow)[4], int lane, int wm, int wn,
                                                int nt, int r0, int seg_end, int fq, int qend, int colq) {
  const bf16* __restrict__ ab = static_cast<const bf16*>(p.ab);
  const int F = p.F, f2s = 2 * F / 32;
  // a and b of the lane's 8 rows of a 32-row block. The 8 blocks (4 per pass) are processed in
  // order, and row s of the next block is loaded into row s's registers as soon as they are
  // unpacked, so those loads run during the rest of the current block.
  uint4 araw[8], braw[8];
  auto load_ab = [&](int i, int s) {
    const int rl = (lane >> 4) + 4 * s, c0 = (lane & 15) * 8;
    const int r = r0 + 128 * wm + 32 * i + rl, f = fq + c0;
    const bf16* abr = ab + (size_t)min(r, seg_end - 1) * 2 * F + min(f, F - 8);
    araw[s] = ld16(abr);
    braw[s] = ld16(abr + F);
  };
  // rows past the segment and columns past F computed from clamped loads, then zeroed
  auto dswiglu = [&](int i, int s, int inext, float (&da)[8], float (&db)[8], float& gsum) {
    const int rl = (lane >> 4) + 4 * s, c0 = (lane & 15) * 8;
    const float wt = __shfl(wrow[i], rl);
    const int r = r0 + 128 * wm + 32 * i + rl, f = fq + c0;
    const bool ok = r < seg_end && f < F;
    float u[8], av[8], bv[8];
    read8(slab, rl, c0, u);
    unpack8(araw[s], av);
    unpack8(braw[s], bv);
    if (inext >= 0) load_ab(inext, s);
    gsum = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float sg = sigmoidf_(av[e]), si = av[e] * sg;
      gsum += u[e] * (si * bv[e]);
      const float dh = wt * u[e];
      da[e] = ok ? dh * bv[e] * sg * (1.0f + av[e] * (1.0f - sg)) : 0.f;
      db[e] = ok ? dh * si : 0.f;
    }
    gsum = ok ? gsum : 0.f;
  };
  auto put_slabs = [&](int s, const float (&da)[8], const float (&db)[8]) {
    const int rl = (lane >> 4) + 4 * s, c0 = (lane & 15) * 8;
    *reinterpret_cast<float4*>(slab + rl * SLD + c0) = make_float4(da[0], da[1], da[2], da[3]);
    *reinterpret_cast<float4*>(slab + rl * SLD + c0 + 4) = make_float4(da[4], da[5], da[6], da[7]);
    *reinterpret_cast<float4*>(slab2 + rl * SLD + c0) = make_float4(db[0], db[1], db[2], db[3]);
    *reinterpret_cast<float4*>(slab2 + rl * SLD + c0 + 4) = make_float4(db[4], db[5], db[6], db[7]);
  };
  // columns lane and lane + 64 of the da and db slabs, over the wave's 128 rows
  float cm[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < 8; ++s) load_ab(0, s);
  auto pass1 = [&](auto I) {
    constexpr int i = decltype(I)::value;
    stage_rows(slab, acc, i, lane);
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      float da[8], db[8], gsum;
      dswiglu(i, s, (i + 1) & 3, da, db, gsum);   // after block 3 come pass 2's blocks from 0
      const int rl = (lane >> 4) + 4 * s, c0 = (lane & 15) * 8;
      const int r = r0 + 128 * wm + 32 * i + rl, f = fq + c0;
      const int sda = fp8b_exponent(mx_amax_x16(da));
      const int sdb = fp8b_exponent(mx_amax_x16(db));
      if (r < seg_end && f < F) {
        uint8_t* qr = p.dabq + (size_t)r * 2 * F + f;
        *reinterpret_cast<uint2*>(qr) = mx_encode8(da, sda);
        *reinterpret_cast<uint2*>(qr + F) = mx_encode8(db, sdb);
        if ((lane & 3) == 0) {
          uint8_t* sr = p.dabs + (size_t)r * f2s;
          sr[f / 32] = (uint8_t)(sda + 127);
          sr[(F + f) / 32] = (uint8_t)(sdb + 127);
        }
      }
      put_slabs(s, da, db);
      gsum = group_sum16(gsum);
      if (r < seg_end && (lane & 15) == 0) p.gpart[(size_t)(nt * 2 + wn) * p.rows + r] = gsum;
    }
    cm[0] = fmaxf(cm[0], column_amax(slab, lane));
    cm[1] = fmaxf(cm[1], column_amax(slab, lane + 64));
    cm[2] = fmaxf(cm[2], column_amax(slab2, lane));
    cm[3] = fmaxf(cm[3], column_amax(slab2, lane + 64));
  };
  pass1(std::integral_constant<int, 0>{});
  pass1(std::integral_constant<int, 1>{});
  pass1(std::integral_constant<int, 2>{});
  pass1(std::integral_constant<int, 3>{});
  const int sc[4] = {fp8b_exponent(cm[0]), fp8b_exponent(cm[1]), fp8b_exponent(cm[2]), fp8b_exponent(cm[3])};
  auto pass2 = [&](auto I) {
    constexpr int i = decltype(I)::value;
    stage_rows(slab, acc, i, lane);
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      float da[8], db[8], gsum;
      dswiglu(i, s, i < 3 ? i + 1 : -1, da, db, gsum);
      put_slabs(s, da, db);
    }
    const int colb = colq + 32 * i;
    store_transposed_fixed(
        slab, lane, 128,
        [&](int c) { return colb < qend && fq + c < F ? p.dabtq + (size_t)(fq + c) * p.qc + colb : nullptr; },
        [&](int c) { return p.dabts + tscale_at(2 * F, fq + c, colb); }, [&](int c) { return c < 64 ? sc[0] : sc[1]; });
    store_transposed_fixed(
        slab2, lane, 128,
        [&](int c) { return colb < qend && fq + c < F ? p.dabtq + (size_t)(F + fq + c) * p.qc + colb : nullptr; },
        [&](int c) { return p.dabts + tscale_at(2 * F, F + fq + c, colb); },
        [&](int c) { return c < 64 ? sc[2] : sc[3]; });
  };
  pass2(std::integral_constant<int, 0>{});
  pass2(std::integral_constant<int, 1>{});
  pass2(std::integral_constant<int, 2>{});
  pass2(std::integral_constant<int, 3>{});
}

template <bool BLK>
__global__ __launch_bounds__(NTHR, 1) void k_bwd_dh_mx(BwdParams p) {
  MX_SMEM
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, wm = w >> 1, wn = w & 1;
  const bf16* __restrict__ ab = static_cast<const bf16*>(p.ab);
  const int H = p.H, F = p.F, ntn = (F + TILE - 1) / TILE, hs = H / 32, f2s = 2 * F / 32;
  const XcdRange xr = xcd_range(*p.num_mtiles2 * ntn);
  const int bn[4] = {128 * wn, 128 * wn + 32, 128 * wn + 64, 128 * wn + 96};
  const int row_s = 128 * sc_half() + 32 * sc_blk() + sc_row32();
  for (int tile = xr.first; tile < xr.end; tile += xr.stride) {
    const int mt = tile / ntn, nt = tile - mt * ntn;
    const int2 me = p.mtile2[mt];
    const int e = me.x, r0 = me.y, seg_end = p.offsets[e + 1];
    KOp la, lb;
#pragma unroll
    for (int j = 0; j < LOADS; ++j) {
      const int row = KOp::row_of(j), c = KOp::chunk_of(j);
      const int r = min(r0 + row, seg_end - 1);
      la.p[j] = reinterpret_cast<const char*>(p.dyq + (size_t)p.ptok[r] * H) + 16 * c;
      const int f = min(nt * TILE + row, F - 1);
      lb.p[j] = reinterpret_cast<const char*>(p.wdtq + ((size_t)e * F + f) * H) + 16 * c;
    }
    const SOp sa{p.dys + (size_t)p.ptok[min(r0 + row_s, seg_end - 1)] * hs, 0};
    const SOp sb{p.wdts + ((size_t)e * F + min(nt * TILE + row_s, F - 1)) * hs, 0};
    int prow[4];   // slots of the wave's rows; their routing weights are loaded after the main loop
#pragma unroll
    for (int i = 0; i < 4; ++i) prow[i] = p.perm[min(r0 + 128 * wm + acc_m(i, lane), seg_end - 1)];
    f32x16 acc[4][4];
    mainloop_mx(acc, smem, la, lb, sa, sb, H / KTILE, 128 * wm, bn, wm, wn);
    float wrow[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) wrow[i] = p.weight[prow[i]];
    float* slab = wave_slab(smem);
    float* slab2 = slab + 4 * SLAB;
    const int fq = nt * TILE + 128 * wn;
    const int qend = p.qoff[e + 1];
    const int colq = p.qoff[e] + (r0 - p.offsets[e]) + 128 * wm;
    if constexpr (BLK) {
      epilogue_dh_blk(p, acc, slab, slab2, wrow, lane, wm, wn, nt, r0, seg_end, fq, qend, colq);
      continue;
    }
    // one 32-row block of the quadrant; i is a compile-time constant so that acc stays in registers
    // a/b of the lane's 8 rows of a 32-row block. Row s of block i+1 is loaded into the registers of
    // row s of block i as soon as those are unpacked, so the next block's loads run during the rest
    // of this block (no extra registers).
    uint4 araw[8], braw[8];
    auto load_ab = [&](int i, int s) {
      const int rl = (lane >> 4) + 4 * s, c0 = (lane & 15) * 8;
      const int r = r0 + 128 * wm + 32 * i + rl, f = fq + c0;
      const bf16* abr = ab + (size_t)min(r, seg_end - 1) * 2 * F + min(f, F - 8);
      araw[s] = ld16(abr);
      braw[s] = ld16(abr + F);
    };
#pragma unroll
    for (int s = 0; s < 8; ++s) load_ab(0, s);
    auto block = [&](auto I) {
      constexpr int i = decltype(I)::value;
      stage_rows(slab, acc, i, lane);
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const int rl = (lane >> 4) + 4 * s, c0 = (lane & 15) * 8;
        const float wt = __shfl(wrow[i], rl);
        const int r = r0 + 128 * wm + 32 * i + rl, f = fq + c0;
        const bool ok = r < seg_end && f < F;
        float gsum = 0.f, da[8], db[8];
        if (ok) {
          float u[8], av[8], bv[8];
          read8(slab, rl, c0, u);
          unpack8(araw[s], av);
          unpack8(braw[s], bv);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float sg = sigmoidf_(av[e]), si = av[e] * sg;
            gsum += u[e] * (si * bv[e]);
            const float dh = wt * u[e];
            da[e] = dh * bv[e] * sg * (1.0f + av[e] * (1.0f - sg));
            db[e] = dh * si;
          }
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) da[e] = db[e] = 0.f;
        }
        if (i < 3) load_ab(i + 1, s);
        const int sda = mx_exponent(mx_amax_x4(da));
        const int sdb = mx_exponent(mx_amax_x4(db));
        if (ok) {
          uint8_t* qr = p.dabq + (size_t)r * 2 * F + f;
          *reinterpret_cast<uint2*>(qr) = mx_encode8(da, sda);
          *reinterpret_cast<uint2*>(qr + F) = mx_encode8(db, sdb);
          if ((lane & 3) == 0) {
            uint8_t* sr = p.dabs + (size_t)r * f2s;
            sr[f / 32] = (uint8_t)(sda + 127);
            sr[(F + f) / 32] = (uint8_t)(sdb + 127);
          }
        }
        *reinterpret_cast<float4*>(slab + rl * SLD + c0) = make_float4(da[0], da[1], da[2], da[3]);
        *reinterpret_cast<float4*>(slab + rl * SLD + c0 + 4) = make_float4(da[4], da[5], da[6], da[7]);
        *reinterpret_cast<float4*>(slab2 + rl * SLD + c0) = make_float4(db[0], db[1], db[2], db[3]);
        *reinterpret_cast<float4*>(slab2 + rl * SLD + c0 + 4) = make_float4(db[4], db[5], db[6], db[7]);
        gsum = group_sum16(gsum);
        if (r < seg_end && (lane & 15) == 0) p.gpart[(size_t)(nt * 2 + wn) * p.rows + r] = gsum;
      }
      const int colb = colq + 32 * i;
      store_transposed_mx(
          slab, lane, 128,
          [&](int c) { return colb < qend && fq + c < F ? p.dabtq + (size_t)(fq + c) * p.qc + colb : nullptr; },
          [&](int c) { return p.dabts + tscale_at(2 * F, fq + c, colb); });
      store_transposed_mx(
          slab2, lane, 128,
          [&](int c) { return colb < qend && fq + c < F ? p.dabtq + (size_t)(F + fq + c) * p.qc + colb : nullptr; },
          [&](int c) { return p.dabts + tscale_at(2 * F, F + fq + c, colb); });
    };
    block(std::integral_constant<int, 0>{});
    block(std::integral_constant<int, 1>{});
    block(std::integral_constant<int, 2>{});
    block(std::integral_constant<int, 3>{});
  }
}

// backward: dX' = [da db] [W_gate[e]; W_up[e]] (contraction over 2F; B = [W_gate^T W_up^T] quantised
// along F, one H x 2F matrix per expert)
__global__ __launch_bounds__(NTHR, 1) void k_dgrad_x_mx(BwdParams p) {
  MX_SMEM
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, wm = w >> 1, wn = w & 1;
  bf16* __restrict__ dxp = static_cast<bf16*>(p.dxp);
  const int H = p.H, F = p.F, ntn = H / TILE, f2s = 2 * F / 32;
  const XcdRange xr = xcd_range(*p.num_mtiles2 * ntn);
  const int bn[4] = {128 * wn, 128 * wn + 32, 128 * wn + 64, 128 * wn + 96};
  const int row_s = 128 * sc_half() + 32 * sc_blk() + sc_row32();
  for (int tile = xr.first; tile < xr.end; tile += xr.stride) {
    const int mt = tile / ntn, nt = tile - mt * ntn;
    const int2 me = p.mtile2[mt];
    const int e = me.x, r0 = me.y, seg_end = p.offsets[e + 1];
    KOp la, lb;
#pragma unroll
    for (int j = 0; j < LOADS; ++j) {
      const int row = KOp::row_of(j), c = KOp::chunk_of(j);
      const int r = min(r0 + row, seg_end - 1);
      la.p[j] = reinterpret_cast<const char*>(p.dabq + (size_t)r * 2 * F) + 16 * c;
      lb.p[j] = reinterpret_cast<const char*>(p.wgutq + ((size_t)e * H + nt * TILE + row) * 2 * F) + 16 * c;
    }
    const SOp sa{p.dabs + (size_t)min(r0 + row_s, seg_end - 1) * f2s, 0};
    const SOp sb{p.wguts + ((size_t)e * H + nt * TILE + row_s) * f2s, 0};
    f32x16 acc[4][4];
    mainloop_mx(acc, smem, la, lb, sa, sb, 2 * F / KTILE, 128 * wm, bn, wm, wn);
    const int rq = r0 + 128 * wm;
    bf16* const oq = dxp + nt * TILE + 128 * wn;
    store_wave_block(smem, acc, lane, [&](int m) { return rq + m < seg_end ? oq + (size_t)(rq + m) * H : nullptr; }, 128);
  }
}

// backward: dW_down[e] (H x F) = sum over the expert's pairs of dY_t hw_r^T. A = dY^T and B = hw^T,
// both pair-contiguous and quantised along the pairs; the expert's K range is its padded segment.
__global__ __launch_bounds__(NTHR, 1) void k_wgrad_down_mx(BwdParams p) {
  MX_SMEM
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, wm = w >> 1, wn = w & 1;
  const int H = p.H, F = p.F, ntn = (F + TILE - 1) / TILE, tpe = (H / TILE) * ntn;
  const XcdRange xr = xcd_range_split(p.sched + kSchedWgradDown * kSchedInts);
  const int bn[4] = {128 * wn, 128 * wn + 32, 128 * wn + 64, 128 * wn + 96};
  const int row_s = 128 * sc_half() + 32 * sc_blk() + sc_row32();
  for (int lid = xr.first; lid < xr.end; lid += xr.stride) {
    const int e = lid / tpe, t = lid - e * tpe, mt = t / ntn, nt = t - mt * ntn;
    const int q0 = p.qoff[e], nk = (p.qoff[e + 1] - q0) / KTILE;
    KOp la, lb;
#pragma unroll
    for (int j = 0; j < LOADS; ++j) {
      const int row = KOp::row_of(j), c = KOp::chunk_of(j);
      la.p[j] = reinterpret_cast<const char*>(p.dytq + (size_t)(mt * TILE + row) * p.qc + q0) + 16 * c;
      lb.p[j] = reinterpret_cast<const char*>(p.hwtq + (size_t)min(nt * TILE + row, F - 1) * p.qc + q0) + 16 * c;
    }
    const SOp sa{p.dyts + tscale_at(H, mt * TILE + row_s, q0), 0, 4 * H};
    const SOp sb{p.hwts + tscale_at(F, min(nt * TILE + row_s, F - 1), q0), 0, 4 * F};
    f32x16 acc[4][4];
    mainloop_mx(acc, smem, la, lb, sa, sb, nk, 128 * wm, bn, wm, wn);
    bf16* __restrict__ out = static_cast<bf16*>(p.dwd) + (size_t)e * H * F;
    const int mq = mt * TILE + 128 * wm, nq = nt * TILE + 128 * wn;
    store_wave_block(smem, acc, lane, [&](int m) { return out + (size_t)(mq + m) * F + nq; }, F - nq);
  }
}

// backward: [dW_gate; dW_up][e] (2F x H) = sum over the expert's pairs of [da; db]_r x_t^T. A = [da db]^T
// and B = x^T, both pair-contiguous and quantised along the pairs.
__global__ __launch_bounds__(NTHR, 1) void k_wgrad_gateup_mx(BwdParams p) {
  MX_SMEM
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, wm = w >> 1, wn = w & 1;
  const int H = p.H, F = p.F, ntn = H / TILE, tpe = (2 * F / TILE) * ntn;
  const XcdRange xr = xcd_range_split(p.sched + kSchedWgradGateup * kSchedInts);
  const int bn[4] = {128 * wn, 128 * wn + 32, 128 * wn + 64, 128 * wn + 96};
  const int row_s = 128 * sc_half() + 32 * sc_blk() + sc_row32();
  for (int lid = xr.first; lid < xr.end; lid += xr.stride) {
    const int e = lid / tpe, t = lid - e * tpe, mt = t / ntn, nt = t - mt * ntn;
    const int q0 = p.qoff[e], nk = (p.qoff[e + 1] - q0) / KTILE;
    KOp la, lb;
#pragma unroll
    for (int j = 0; j < LOADS; ++j) {
      const int row = KOp::row_of(j), c = KOp::chunk_of(j);
      la.p[j] = reinterpret_cast<const char*>(p.dabtq + (size_t)(mt * TILE + row) * p.qc + q0) + 16 * c;
      lb.p[j] = reinterpret_cast<const char*>(p.xtq + (size_t)(nt * TILE + row) * p.qc + q0) + 16 * c;
    }
    const SOp sa{p.dabts + tscale_at(2 * F, mt * TILE + row_s, q0), 0, 8 * F};
    const SOp sb{p.xts + tscale_at(H, nt * TILE + row_s, q0), 0, 4 * H};
    f32x16 acc[4][4];
    mainloop_mx(acc, smem, la, lb, sa, sb, nk, 128 * wm, bn, wm, wn);
    bf16* __restrict__ dwg = static_cast<bf16*>(p.dwg) + (size_t)e * F * H;
    bf16* __restrict__ dwu = static_cast<bf16*>(p.dwu) + (size_t)e * F * H;
    const int mq = mt * TILE + 128 * wm, nq = nt * TILE + 128 * wn;
    store_wave_block(smem, acc, lane, [&](int m) {
      const int mm = mq + m;
      return (mm < F ? dwg + (size_t)mm * H : dwu + (size_t)(mm - F) * H) + nq;
    }, 128);
  }
}

}  // namespace

hipError_t launch_forward_gemms_mx(const FwdParams& p, int grid, hipStream_t s, bool recompute) {
  hipError_t err;
  prof_mark_begin(recompute ? "gemm_gateup_recompute" : "gemm_gateup_swiglu", s);
  if (p.blk)
    k_gateup_mx<true><<<grid, NTHR, 0, s>>>(p);
  else
    k_gateup_mx<false><<<grid, NTHR, 0, s>>>(p);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  prof_mark_end(s);
  if (recompute) return hipSuccess;
  prof_mark_begin("gemm_down", s);
  k_down_mx<<<grid, NTHR, 0, s>>>(p);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  prof_mark_end(s);
  return hipSuccess;
}

// dH, then the dgrad of x, on the caller's stream; the two weight gradients on the device's side
// stream when there is one (the down one from the start, the gate/up one after dH), as in the bf16
// backward
hipError_t launch_backward_gemms_mx(const BwdParams& p, int grid, hipStream_t s) {
  hipError_t err;
  if ((err = launch_sched_setup(p, KTILE, s)) != hipSuccess) return err;
  hipStream_t s1 = side_stream_fork(s);
  hipStream_t sw = s1 ? s1 : s;   // the weight gradients' stream
  prof_mark_begin("gemm_bwd_dh_dswiglu", s);
  if (p.blk)
    k_bwd_dh_mx<true><<<grid, NTHR, 0, s>>>(p);
  else
    k_bwd_dh_mx<false><<<grid, NTHR, 0, s>>>(p);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  prof_mark_end(s);
  if (s1 && (err = side_stream_mark(s)) != hipSuccess) return err;
  prof_mark_begin("gemm_wgrad_down", sw);
  k_wgrad_down_mx<<<grid, NTHR, 0, sw>>>(p);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  prof_mark_end(sw);
  if (s1 && (err = side_stream_wait_mark()) != hipSuccess) return err;
  prof_mark_begin("gemm_wgrad_gateup", sw);
  k_wgrad_gateup_mx<<<grid, NTHR, 0, sw>>>(p);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  prof_mark_end(sw);
  prof_mark_begin("gemm_dgrad_x", s);
  k_dgrad_x_mx<<<grid, NTHR, 0, s>>>(p);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  prof_mark_end(s);
  return hipSuccess;
}

}  // namespace moe
