// bf16 grouped-GEMM engine for gfx950 and the six expert GEMMs of the fused MoE layer.
// The SwiGLU experts and the combine are from "A Magia da Fusão" on "IA: MoE Kernel 3x Mais Rápido
// Chegou!"; the backward pass is from "Afinal, o que é esse Prime Mega MoE?" on the same page;
// the bf16 precision mode is from "Supporto di precisione e vincoli hardware" on "Prime Mega MoE:
// il kernel che accelera il training AI del 55%".
//
// Engine:
//  * A workgroup of 8 wavefronts (2 per SIMD) computes a 256x256 output tile. Each wave owns a
//    64x128 eighth as 2x4 blocks of v_mfma_f32_32x32x16_bf16 with fp32 accumulators (128 per
//    lane), or a 128x64 eighth (4x2 blocks) in the dgrad of h, whose epilogue stages two fp32
//    slabs. With two waves per SIMD one issues MFMAs while the other waits on LDS, its loads or the
//    barrier; this outweighs the extra fragment reads (a wave reads 6 fragments per 8 MFMAs instead
//    of 8 per 16): measured 9 % faster on a dense 8192x8192x2048 product and 20 % at K = 768.
//  * A K-tile is 64 contraction elements. Operand tiles reach LDS with global_load_lds_dwordx4
//    (no VGPR staging) through a 2-stage ring of 64 KB stages: K-tile kt+1 lands while kt is
//    multiplied. Each wave waits for its own loads, then a barrier publishes them.
//  * K-major operand (contraction axis contiguous: x, dY, hw, dab rows, and the weights in the
//    forward): one 128-byte LDS row per M/N index, so every load moves whole cache lines (with
//    64-byte rows the direct-to-LDS path ran at half the bytes per cycle). Chunk c of row r goes
//    to slot c ^ ((r >> 1) & 7). ds_read_b128 fragment reads are then conflict-free.
//  * MN-major operand (M/N axis contiguous: the weights in the dgrad GEMMs, every weight-gradient
//    operand): one 512-byte LDS row per contraction index. Chunk c of row k goes to slot
//    c ^ ((k & 3) << 2). Fragments are read with ds_read_b64_tr_b16, which transposes 16x4
//    blocks on the fly. In each 16-lane group, lane s reads 4 columns of row k0 + s/4; lane i
//    then receives column i of rows k0..k0+3. The four rows of one read land in disjoint bank
//    groups.
//  * Rows outside an expert's segment are clamped to a valid row when they only feed discarded
//    outputs. When they would contribute to a contraction, they read the zero page. The token
//    indices of gathered contraction rows come through scalar loads, so that the vector memory
//    counter tracks nothing but the tile loads.
//  * The kernels are persistent. Each XCD takes one contiguous range of the expert-major tile list,
//    so the blocks sharing an expert's operands share that XCD's L2. The gate/up GEMM and the dgrad
//    of h hand out the tiles of a range dynamically (TileSched), since an expert's last tile may be
//    a half tile (or, for the dgrad of h, multiply fewer row blocks); the others assign them
//    round-robin and issue each tile's first K-tile before the previous tile's epilogue
//    (mainloop_pre): the weight-gradient tiles cost the same within an expert (the dynamic order
//    measured 3-5 % slower there), and the down GEMM's and the dgrad of x's tiles all contract over
//    the same K, the pre-issued K-tile gaining more than the counter's balance of half tiles.

#include "engine.h"
#include "moe_internal.h"

namespace moe {
namespace {

using namespace eng;

constexpr int NWAVE = 8;             // wavefronts per workgroup
constexpr int NTHR8 = 64 * NWAVE;
constexpr int KTILE = 64;            // contraction elements per K-tile: 128 bytes per K-major row
typedef KRows<128, NWAVE> KOp;       // K-major operand loader (8 rows of 128 bytes per wave instruction)
constexpr int LOADS = KOp::LOADS;    // 4 direct-to-LDS loads per lane per operand per K-tile
constexpr int KPW = KTILE / NWAVE;   // contraction rows of an MN-major operand loaded by one wave
constexpr int OPB = 32768;           // bytes per operand per stage (256 x 128 B, or 64 x 512 B)
constexpr int STB = 2 * OPB;         // bytes per stage
constexpr int STAGES = 2;            // LDS ring depth (2 x 64 KB)

__device__ __forceinline__ const char* mn_addr(const char* tile, int k, int col) {
  return tile + k * 512 + ((((col >> 3) ^ ((k & 3) << 2))) << 4) + (col & 7) * 2;
}

__device__ __forceinline__ bf16x8 frag_mn(const char* tile, int col0, int ks, int lane) {
  const int g = lane >> 4, s = lane & 15;
  const int k = 16 * ks + 8 * (g >> 1) + (s >> 2);
  const int col = col0 + 16 * (g & 1) + 4 * (s & 3);
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)mn_addr(tile, k, col));
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)mn_addr(tile, k + 4, col));
  typedef short i16x8 __attribute__((ext_vector_type(8)));
  const i16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, v);
}

// ------------------------------------------------------------------------------------------------
// Operand loaders. issue(stage_tile, kt) starts the LOADS direct-to-LDS loads this lane owns for
// K-tile kt. prefetch(kt) fetches (into SGPRs) the row indices issue(kt) will need; it runs one
// K-tile ahead of issue.

// contraction row owned by this lane in load slot j of an MN-major operand (2 rows per slot)
__device__ __forceinline__ int mn_krow(int j) { return wave_id() * KPW + 2 * j + ((threadIdx.x & 63) >> 5); }

// MN-major operand: 64 contraction rows of 256 columns starting at column col0. This lane owns
// contraction rows w*8 + 2j + lane/32 (j < 4) and slot lane&31. Each wave instruction moves two
// whole 512-byte rows.
template <class Rows>
struct MNOp {
  Rows rows;
  const char* zero;
  int coff[LOADS];     // byte offset of this lane's column chunk, or -1 if past the last column
  __device__ __forceinline__ void init(int col0, int ncols) {
#pragma unroll
    for (int j = 0; j < LOADS; ++j) {
      const int c = (threadIdx.x & 31) ^ ((mn_krow(j) & 3) << 2);
      coff[j] = col0 + 8 * c < ncols ? 16 * c : -1;
    }
  }
  __device__ __forceinline__ void prefetch(int kt) { rows.prefetch(kt); }
  __device__ __forceinline__ void issue(char* tile, int kt) const {
    const int w = wave_id();
#pragma unroll
    for (int j = 0; j < LOADS; ++j) {
      const char* r = rows.row(kt, j);
      gl2lds(r && coff[j] >= 0 ? r + coff[j] : zero, tile + (w * LOADS + j) * 1024);
    }
  }
  // prologue: the row indices of the first STAGES K-tiles are fetched together (kt is a
  // compile-time slot after unrolling), then the tiles are issued
  __device__ __forceinline__ void prologue_prefetch(int kt) { rows.prologue_prefetch(kt); }
  __device__ __forceinline__ void prologue_issue(char* tile, int kt) const {
    const int w = wave_id();
#pragma unroll
    for (int j = 0; j < LOADS; ++j) {
      const char* r = rows.prologue_row(kt, j);
      gl2lds(r && coff[j] >= 0 ? r + coff[j] : zero, tile + (w * LOADS + j) * 1024);
    }
  }
};

// contraction rows of a weight matrix: row k at base + k*ld (k < split) or base2 + (k-split)*ld
struct WeightRows {
  const char* base;
  const char* base2;
  size_t ld;
  int split;
  __device__ __forceinline__ void prefetch(int) {}
  __device__ __forceinline__ void prologue_prefetch(int) {}
  __device__ __forceinline__ const char* row(int kt, int j) const {
    const int k = kt * KTILE + mn_krow(j);
    return k < split ? base + (size_t)k * ld : base2 + (size_t)(k - split) * ld;
  }
  __device__ __forceinline__ const char* prologue_row(int kt, int j) const { return row(kt, j); }
};

// contraction rows = an expert's pairs, as the token rows of a [T, ld] tensor (ptok maps a
// sorted pair to its token). The wave's 8 token indices of a K-tile arrive through scalar loads.
struct GatherRows {
  const char* base;
  const int* __restrict__ ptok;
  size_t ld;
  int seg0, seg_end;
  int tok[KPW];
  int tokp[STAGES][KPW];   // prologue K-tiles
  __device__ __forceinline__ void prefetch(int kt) {
    const int r0 = seg0 + kt * KTILE + wave_id() * KPW;
#pragma unroll
    for (int i = 0; i < KPW; ++i) tok[i] = ld_uniform(ptok, min(r0 + i, seg_end - 1));
  }
  __device__ __forceinline__ void prologue_prefetch(int kt) {
    const int r0 = seg0 + kt * KTILE + wave_id() * KPW;
#pragma unroll
    for (int i = 0; i < KPW; ++i) tokp[kt][i] = ld_uniform(ptok, min(r0 + i, seg_end - 1));
  }
  __device__ __forceinline__ const char* row(int kt, int j) const {
    const int hi = (threadIdx.x & 63) >> 5;
    const int r = seg0 + kt * KTILE + mn_krow(j);
    const int t = hi ? tok[2 * j + 1] : tok[2 * j];
    return r < seg_end ? base + (size_t)t * ld : nullptr;
  }
  __device__ __forceinline__ const char* prologue_row(int kt, int j) const {
    const int hi = (threadIdx.x & 63) >> 5;
    const int r = seg0 + kt * KTILE + mn_krow(j);
    const int t = hi ? tokp[kt][2 * j + 1] : tokp[kt][2 * j];
    return r < seg_end ? base + (size_t)t * ld : nullptr;
  }
};

// ------------------------------------------------------------------------------------------------
// Main loop: nk K-tiles, accumulating into the wave's MI x NJ blocks acc. A fragments from rows
// am0 + 32i of the A tile; B fragments from columns bn[j]. A K-tile is four 16-deep steps; each step's fragments are read
// while the previous step's MFMAs run. The ring holds two K-tiles: K-tile kt+1 lands while kt is
// multiplied. After the last fragments of K-tile kt are read, the wave waits for K-tile kt+1, the
// barrier publishes it and frees kt's stage, A's part of K-tile kt+2 is issued into that stage
// (with B's part when B is K-major), and the first fragments of kt+1 are read while the last MFMAs
// of kt run; an MN-major B's part of K-tile kt+2 follows those MFMAs. On return all LDS reads are
// done (LDS may be reused).
__device__ __forceinline__ bf16x8 frag_k(const char* tile, int row0, int ks, int lane) {
  return *reinterpret_cast<const bf16x8*>(KOp::at(tile, row0 + (lane & 31), 2 * ks + (lane >> 5)));
}

// A fragments of the first NA row blocks (rows am0 + AST i), B fragments of every column block
template <bool AMN, bool BMN, int AST, int NA, int MI, int NJ>
__device__ __forceinline__ void read_frags(bf16x8 (&fa)[MI], bf16x8 (&fb)[NJ], const char* st, int ks, int am0,
                                           const int (&bn)[NJ], int lane) {
#pragma unroll
  for (int i = 0; i < NA; ++i) fa[i] = AMN ? frag_mn(st, am0 + AST * i, ks, lane) : frag_k(st, am0 + AST * i, ks, lane);
  if (NA > 0) {   // a wave with no active row block multiplies nothing
#pragma unroll
    for (int j = 0; j < NJ; ++j) fb[j] = BMN ? frag_mn(st + OPB, bn[j], ks, lane) : frag_k(st + OPB, bn[j], ks, lane);
  }
}

// The B fragment is passed as the MFMA's first operand, so each accumulator block holds the
// transposed 32x32 block: lane l keeps row (l & 31) of C and 4 consecutive columns per group of 4.
template <int NA, int MI, int NJ>
__device__ __forceinline__ void mma_step(f32x16 (&acc)[MI][NJ], const bf16x8 (&fa)[MI], const bf16x8 (&fb)[NJ]) {
#pragma unroll
  for (int i = 0; i < NA; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[j], fa[i], acc[i][j], 0, 0, 0);
  // issue order: one MFMA, then one of the next step's LDS fragment reads, and so on, so that the
  // reads spread over the step instead of reaching the LDS port in one burst (the weight gradients
  // and the dgrad measured 2-4 % faster than with the compiler's own grouping)
#pragma unroll
  for (int q = 0; q < NA * NJ; ++q) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
}

template <bool AMN, bool BMN, int AST, int ACT, int MI, int NJ, class LA, class LB>
__device__ __forceinline__ void mainloop_body(f32x16 (&acc)[MI][NJ], char* smem, LA& la, LB& lb, int nk, int am0,
                                              const int (&bn)[NJ], bool skip_a);

// Row block i of the wave's A rows starts at am0 + AST i. Only the first NA row blocks run (NA < MI:
// the rows of the others are known to be past the segment; their accumulators stay zero); NA = 0
// runs all MI, NA = -1 none (the wave still loads its share of the operand tiles).
// The waves 4-7 load the A rows from 128 on (K-major A). When no wave needs them they skip those
// loads and wait for their B loads only: skip_hi = 1 or 0 says whether that is so; by default
// (skip_hi = -1) it is taken to be so whenever NA < MI (the row-tiled kernels' half tiles).
template <bool AMN, bool BMN, int AST = 32, int NA = 0, int MI, int NJ, class LA, class LB>
__device__ __forceinline__ void mainloop(f32x16 (&acc)[MI][NJ], char* smem, LA& la, LB& lb, int nk, int am0,
                                         const int (&bn)[NJ], int skip_hi = -1) {
  constexpr int ACT = NA == 0 ? MI : (NA < 0 ? 0 : NA);
  static_assert(ACT == MI || !AMN, "half tiles take a K-major A");
  const bool skip_a = (skip_hi < 0 ? ACT < MI : skip_hi > 0) && wave_id() >= NWAVE / 2;
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;
  if (nk <= 0) return;
  wait_vm<0>();   // stores of the previous tile's epilogue must not count against the ring below
  block_sync();   // and every wave is done reading its epilogue staging slab
#pragma unroll
  for (int s = 0; s < STAGES; ++s) {
    la.prologue_prefetch(s);
    lb.prologue_prefetch(s);
  }
  if (!skip_a) la.prologue_issue(smem, 0);
  lb.prologue_issue(smem + OPB, 0);
  if (nk > 1) {
    if (!skip_a) la.prologue_issue(smem + STB, 1);
    lb.prologue_issue(smem + STB + OPB, 1);
    if (nk > 2) {
      la.prefetch(2);
      lb.prefetch(2);
    }
    // K-tile 0 landed; K-tile 1 may still be in flight
    if (skip_a) wait_vm<LOADS>();
    else wait_vm<2 * LOADS>();
  } else {
    wait_vm<0>();
  }
  block_sync();
  mainloop_body<AMN, BMN, AST, ACT>(acc, smem, la, lb, nk, am0, bn, skip_a);
}

// The K-tile loop once K-tiles 0 and 1 are issued (and K-tile 2's indices prefetched) and K-tile 0
// is published: ACT active row blocks, A's loads skipped when skip_a.
template <bool AMN, bool BMN, int AST, int ACT, int MI, int NJ, class LA, class LB>
__device__ __forceinline__ void mainloop_body(f32x16 (&acc)[MI][NJ], char* smem, LA& la, LB& lb, int nk, int am0,
                                              const int (&bn)[NJ], bool skip_a) {
  const int lane = threadIdx.x & 63;
  bf16x8 fa0[MI], fb0[NJ], fa1[MI], fb1[NJ];
  read_frags<AMN, BMN, AST, ACT>(fa0, fb0, smem, 0, am0, bn, lane);
  for (int kt = 0; kt < nk; ++kt) {
    char* cur = smem + (kt & 1) * STB;
    read_frags<AMN, BMN, AST, ACT>(fa1, fb1, cur, 1, am0, bn, lane);
    mma_step<ACT>(acc, fa0, fb0);
    read_frags<AMN, BMN, AST, ACT>(fa0, fb0, cur, 2, am0, bn, lane);
    mma_step<ACT>(acc, fa1, fb1);
    read_frags<AMN, BMN, AST, ACT>(fa1, fb1, cur, 3, am0, bn, lane);
    mma_step<ACT>(acc, fa0, fb0);
    if (kt + 1 < nk) {
      wait_vm<0>();   // K-tile kt+1 (the only tile in flight) has landed
      block_sync();
      if (kt + 2 < nk) {
        if (!skip_a) la.issue(cur, kt + 2);
        if (kt + 3 < nk) la.prefetch(kt + 3);
        if (!BMN) {
          lb.issue(cur + OPB, kt + 2);
          if (kt + 3 < nk) lb.prefetch(kt + 3);
        }
      }
      read_frags<AMN, BMN, AST, ACT>(fa0, fb0, smem + ((kt + 1) & 1) * STB, 0, am0, bn, lane);
    }
    mma_step<ACT>(acc, fa1, fb1);
    // A K-major B's loads of K-tile kt+2 go out with A's, right after the barrier; an MN-major B's
    // after the last MFMA step. Each order measured 3-5 % faster on the GEMMs it is used for than
    // the other (MN-major B fragments come through the slower transposing LDS read).
    if (BMN && kt + 2 < nk) {
      lb.issue(cur + OPB, kt + 2);
      if (kt + 3 < nk) lb.prefetch(kt + 3);
    }
  }
  block_sync();
}

// epilogue staging: one 64-column slab per wave plus a second one (dgrad of h), or one 128-column slab
constexpr int SLABS_BYTES = 2 * NWAVE * Stage<2>::SIZE * 4 > NWAVE * Stage<4>::SIZE * 4 ? 2 * NWAVE * Stage<2>::SIZE * 4
                                                                                      : NWAVE * Stage<4>::SIZE * 4;
// Row-tiled kernels: the wave's row blocks are interleaved (block i at tile row am0 + AST i, with
// AST x MI = 256), so that the first 128 rows of the tile are the first MI/2 blocks of every wave.
// An expert's last tile with at most 128 valid rows (half tile) runs only those: each wave does
// half the MFMAs.
template <bool AMN, bool BMN, int AST, int MI, int NJ, class LA, class LB>
__device__ __forceinline__ void mainloop_rows(f32x16 (&acc)[MI][NJ], char* smem, LA& la, LB& lb, int nk, int am0,
                                              const int (&bn)[NJ], bool half) {
  static_assert(AST * MI == TILE, "row blocks");
  if (half) mainloop<AMN, BMN, AST, MI / 2>(acc, smem, la, lb, nk, am0, bn);
  else mainloop<AMN, BMN, AST, MI>(acc, smem, la, lb, nk, am0, bn);
}

constexpr int SMEM_BYTES = STAGES * STB > SLABS_BYTES ? STAGES * STB : SLABS_BYTES;
static_assert(SMEM_BYTES <= 160 * 1024, "LDS");
#define MOE_SMEM __shared__ __attribute__((aligned(1024))) char smem[SMEM_BYTES];

// Persistent tiles with the next tile's first K-tile issued before the current tile's epilogue:
// the caller issues K-tile 0 of a tile into stage 0 (after the previous main loop's last barrier,
// before the previous epilogue), and stages that epilogue in bf16 in stage 1. mainloop_pre then
// waits for every wave's staging reads, issues K-tile 1 into stage 1 and waits for K-tile 0 only,
// so K-tile 0's latency and the epilogue's stores overlap. after_stores says whether this wave
// issued its NS epilogue stores after K-tile 0 (false for its first tile): the vector-memory counter
// completes in order, so K-tile 0 has landed once at most NS stores and K-tile 1's loads remain.
template <int NS, bool AMN, bool BMN, int MI, int NJ, class LA, class LB>
__device__ __forceinline__ void mainloop_pre(f32x16 (&acc)[MI][NJ], char* smem, LA& la, LB& lb, int nk, int am0,
                                             const int (&bn)[NJ], bool after_stores) {
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;
  if (nk <= 0) return;
  block_sync();   // every wave is done reading its staging area in stage 1
  if (nk > 1) {
    la.prologue_prefetch(1);
    lb.prologue_prefetch(1);
    la.prologue_issue(smem + STB, 1);
    lb.prologue_issue(smem + STB + OPB, 1);
    if (nk > 2) {
      la.prefetch(2);
      lb.prefetch(2);
    }
    if (after_stores) wait_vm<NS + 2 * LOADS>();
    else wait_vm<2 * LOADS>();
  } else {
    if (after_stores) wait_vm<NS>();
    else wait_vm<0>();
  }
  block_sync();
  mainloop_body<AMN, BMN, 32, MI>(acc, smem, la, lb, nk, am0, bn, false);
}

// K-tile 0 of a tile into stage 0 (its row indices first); skip_a: this wave loads no A rows (the
// upper waves of a half tile)
template <class LA, class LB>
__device__ __forceinline__ void issue_k0(char* smem, LA& la, LB& lb, bool skip_a = false) {
  la.prologue_prefetch(0);
  lb.prologue_prefetch(0);
  if (!skip_a) la.prologue_issue(smem, 0);
  lb.prologue_issue(smem + OPB, 0);
}

// mainloop_pre for the row-tiled kernels (row block i of the wave at am0 + AST i, as in
// mainloop_rows): a half tile runs only the first MI/2 row blocks, and its waves 4-7 load no A rows
// (issue_k0 with skip_a for its K-tile 0). after_stores is true only when exactly NS stores were
// issued after K-tile 0; otherwise the wait also covers whatever stores preceded K-tile 1.
template <int NS, bool AMN, bool BMN, int AST, int MI, int NJ, class LA, class LB>
__device__ __forceinline__ void mainloop_pre_rows(f32x16 (&acc)[MI][NJ], char* smem, LA& la, LB& lb, int nk, int am0,
                                                  const int (&bn)[NJ], bool after_stores, bool half) {
  static_assert(AST * MI == TILE && !AMN, "row blocks, K-major A");
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;
  if (nk <= 0) return;
  const bool skip_a = half && wave_id() >= NWAVE / 2;
  block_sync();   // every wave is done reading its staging area in stage 1
  if (nk > 1) {
    la.prologue_prefetch(1);
    lb.prologue_prefetch(1);
    if (!skip_a) la.prologue_issue(smem + STB, 1);
    lb.prologue_issue(smem + STB + OPB, 1);
    if (nk > 2) {
      la.prefetch(2);
      lb.prefetch(2);
    }
    // K-tile 0 has landed once only the stores after it (NS or none) and K-tile 1 remain
    if (skip_a) {
      if (after_stores) wait_vm<NS + LOADS>();
      else wait_vm<LOADS>();
    } else {
      if (after_stores) wait_vm<NS + 2 * LOADS>();
      else wait_vm<2 * LOADS>();
    }
  } else {
    if (after_stores) wait_vm<NS>();
    else wait_vm<0>();
  }
  block_sync();
  if (half) mainloop_body<AMN, BMN, AST, MI / 2>(acc, smem, la, lb, nk, am0, bn, skip_a);
  else mainloop_body<AMN, BMN, AST, MI>(acc, smem, la, lb, nk, am0, bn, false);
}

// store_wave_block_bf16 (engine.h) with its staging in ring stage 1, so that stage 0 can take the
// next tile's first K-tile meanwhile (32 rows at a time: 4.6 KB per wave for NJ = 2; 16 rows: 4.4 KB
// for NJ = 4)
template <int MI, int NJ, int RS = 32, class OutRow>
__device__ __forceinline__ void store_wave_block_s1(char* smem, const f32x16 (&acc)[MI][NJ], int lane, OutRow out_row,
                                                    int ncols = 32 * NJ) {
  static_assert(NWAVE * RS * (32 * NJ + 8) * 2 <= STB, "the staging fits ring stage 1");
  store_wave_block_bf16<MI, NJ, RS>(smem + STB, acc, lane, out_row, ncols);
}

// ------------------------------------------------------------------------------------------------
// forward: [a | b] = gather(x) [W_gate; W_up]^T, then ab and hw = w * silu(a) * b
// QT: the pair-contiguous copy of hw is written as MXFP8 (blocks of 32 along the pairs, quantised
// from the fp32 values) for an MXFP8 backward, instead of bf16
// Each output may be null, and is then not written: under activation checkpointing the forward
// writes hw alone (for the down GEMM), and the backward's recompute ab and the transposed copy.
template <bool QT>
__global__ __launch_bounds__(NTHR8, 1) void k_gateup_bf16(FwdParams p) {
  MOE_SMEM
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, wm = w >> 1, wn = w & 1;   // 64x128 per wave
  const bf16* __restrict__ x = static_cast<const bf16*>(p.x);
  const bf16* __restrict__ wg = static_cast<const bf16*>(p.wg);
  const bf16* __restrict__ wu = static_cast<const bf16*>(p.wu);
  bf16* __restrict__ ab = static_cast<bf16*>(p.ab);
  bf16* __restrict__ hw = static_cast<bf16*>(p.hw);
  const int H = p.H, F = p.F, ntn = F / 128;
  __shared__ int s_tile;
  TileSched ts(p.sched + 0 * kSchedInts, *p.num_mtiles2 * ntn);
  const int bn[4] = {64 * wn, 64 * wn + 32, 128 + 64 * wn, 128 + 64 * wn + 32};
  for (int tile = ts.first(&s_tile); tile >= 0; tile = ts.next(&s_tile)) {
    const int mt = tile / ntn, nt = tile - mt * ntn;
    const int2 me = p.mtile2[mt];
    const int e = me.x, r0 = me.y, seg_end = p.offsets[e + 1];
    KOp la, lb;
#pragma unroll
    for (int j = 0; j < LOADS; ++j) {
      const int row = KOp::row_of(j), c = KOp::chunk_of(j);
      const int r = min(r0 + row, seg_end - 1);
      la.p[j] = reinterpret_cast<const char*>(x + (size_t)p.ptok[r] * H) + 16 * c;
      const bf16* wrow = row < 128 ? wg + ((size_t)e * F + nt * 128 + row) * H : wu + ((size_t)e * F + nt * 128 + row - 128) * H;
      lb.p[j] = reinterpret_cast<const char*>(wrow) + 16 * c;
    }
    // routing weight of tile row 32 wm + 128 i + (lane & 31): the slot index is loaded before the
    // main loop, the weight it selects after it, so that no dependent pair of loads sits ahead of
    // the first K-tile's loads (the MXFP8 gate/up GEMM measured 0.8 % faster; bf16 unchanged)
    int prow[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) prow[i] = p.perm[min(r0 + 32 * wm + 128 * i + (lane & 31), seg_end - 1)];
    f32x16 acc[2][4];
    mainloop_rows<false, false, 128>(acc, smem, la, lb, H / KTILE, 32 * wm, bn, seg_end - r0 <= 128);
    ts.fetch();
    float wrow[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) wrow[i] = p.weight[prow[i]];
    // staged columns 0..63 hold gate columns f0.., 64..127 the matching up columns. After the row
    // pass the gate columns hold hw (zero on rows past the segment), which is then written to the
    // pair-contiguous copy hwT[f][qoff[e] + pair - offsets[e]] as well.
    float* slab = wave_slab(smem);
    const int f0 = nt * 128 + 64 * wn;
    bf16* __restrict__ hwt = static_cast<bf16*>(p.hwt);
    const int qend = p.qoff[e + 1];
    const int colq = p.qoff[e] + (r0 - p.offsets[e]) + 32 * wm;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      stage_rows(slab, acc, i, lane);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int rl = (lane >> 3) + 8 * s, c0 = (lane & 7) * 8;
        const float wt = __shfl(wrow[i], rl);
        const int r = r0 + 32 * wm + 128 * i + rl;
        float hv[8];
        if (r < seg_end) {
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
          if (hw) st16_nt(hw + (size_t)r * F + f0 + c0, pack8(hv));
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) hv[e] = 0.f;
        }
        *reinterpret_cast<float4*>(slab + rl * SLD + c0) = make_float4(hv[0], hv[1], hv[2], hv[3]);
        *reinterpret_cast<float4*>(slab + rl * SLD + c0 + 4) = make_float4(hv[4], hv[5], hv[6], hv[7]);
      }
      const int colb = colq + 128 * i;
      if (QT)   // (selected only with a copy to write)
        store_transposed_mx(
            slab, lane, 64, [&](int c) { return colb < qend ? p.hwtq + (size_t)(f0 + c) * p.qc + colb : nullptr; },
            [&](int c) { return p.hwts + tscale_at(F, f0 + c, colb); });
      else if (hwt)
        store_transposed(slab, lane, 64, [&](int c) { return colb < qend ? hwt + (size_t)(f0 + c) * p.qc + colb : nullptr; });
    }
  }
}

// forward: o' = hw W_down[e]^T
// Static per-XCD tile ranges taken round-robin (every tile contracts over F, so equal counts
// balance), each tile's first K-tile issued before the previous tile's epilogue, which stages its
// rows as bf16 in ring stage 1, 16 at a time (mainloop_pre_rows, store_wave_block_s1).
__global__ __launch_bounds__(NTHR8, 1) void k_down_bf16(FwdParams p) {
  MOE_SMEM
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, wm = w >> 1, wn = w & 1;   // 64x128 per wave
  const bf16* __restrict__ hw = static_cast<const bf16*>(p.hw);
  const bf16* __restrict__ wd = static_cast<const bf16*>(p.wd);
  bf16* __restrict__ o = static_cast<bf16*>(p.o);
  const int H = p.H, F = p.F, ntn = H / TILE, nk = F / KTILE;
  const XcdRange xr = xcd_range(ld_uniform(p.num_mtiles2, 0) * ntn);
  const int bn[4] = {128 * wn, 128 * wn + 32, 128 * wn + 64, 128 * wn + 96};
  KOp la, lb;
  int r0 = 0, seg_end = 0, nt = 0;
  bool half = false;
  // loaders of tile `tile` (scalar loads for the tables: see dgrad_x_tiles_pre)
  auto setup = [&](int tile) {
    const int mt = tile / ntn;
    nt = tile - mt * ntn;
    const int e = ld_uniform(reinterpret_cast<const int*>(p.mtile2), 2 * mt);
    r0 = ld_uniform(reinterpret_cast<const int*>(p.mtile2), 2 * mt + 1);
    seg_end = ld_uniform(p.offsets, e + 1);
    half = seg_end - r0 <= 128;
#pragma unroll
    for (int j = 0; j < LOADS; ++j) {
      const int row = KOp::row_of(j), c = KOp::chunk_of(j);
      const int r = min(r0 + row, seg_end - 1);
      la.p[j] = reinterpret_cast<const char*>(hw + (size_t)r * F) + 16 * c;
      lb.p[j] = reinterpret_cast<const char*>(wd + ((size_t)e * H + nt * TILE + row) * F) + 16 * c;
    }
  };
  constexpr int NS = 2 * 32 * 16 / 64;   // epilogue stores per lane of a full tile (MI = 2, NJ = 4)
  int lid = xr.first;
  if (lid >= xr.end) return;
  setup(lid);
  issue_k0(smem, la, lb, half && wave_id() >= NWAVE / 2);
  bool after_stores = false;
  for (; lid < xr.end; lid += xr.stride) {
    f32x16 acc[2][4];
    mainloop_pre_rows<NS, false, false, 128>(acc, smem, la, lb, nk, 32 * wm, bn, after_stores, half);
    const int cr0 = r0, cseg = seg_end, cnt = nt;
    // every wave is past the main loop's last barrier: stage 0 is free
    after_stores = false;
    if (lid + xr.stride < xr.end) {
      setup(lid + xr.stride);
      issue_k0(smem, la, lb, half && wave_id() >= NWAVE / 2);
      after_stores = cseg - cr0 >= TILE;   // every row of the tile is stored: NS stores follow
    }
    const int rq = cr0 + 32 * wm;   // the wave's row m is tile row 32 wm + 128 (m / 32) + m % 32
    bf16* const oq = o + cnt * TILE + 128 * wn;
    store_wave_block_s1<2, 4, 16>(smem, acc, lane, [&](int m) {
      const int r = rq + 128 * (m >> 5) + (m & 31);
      return r < cseg ? oq + (size_t)r * H : nullptr;
    });
  }
}

// backward: u = gather(dY) W_down[e]; epilogue writes g partials, da, db
// One tile of each backward GEMM. fetch() runs once, right after the tile's main loop (a dynamic
// scheduler's counter increment, whose latency then hides behind the epilogue; or nothing).
template <class Fetch>
__device__ __forceinline__ void dh_tile(const BwdParams& p, char* smem, int tile, Fetch fetch) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, wm = w >> 2, wn = w & 3;   // 128x64 per wave
  const bf16* __restrict__ dy = static_cast<const bf16*>(p.dy);
  const bf16* __restrict__ ab = static_cast<const bf16*>(p.ab);
  bf16* __restrict__ dab = static_cast<bf16*>(p.dab);
  const int H = p.H, F = p.F, ntn = (F + TILE - 1) / TILE;
  const int bn[2] = {64 * wn, 64 * wn + 32};
  {
    const int mt = tile / ntn, nt = tile - mt * ntn;
    const int2 me = p.mtile2[mt];
    const int e = me.x, r0 = me.y, seg_end = p.offsets[e + 1];
    KOp la;
#pragma unroll
    for (int j = 0; j < LOADS; ++j) {
      const int r = min(r0 + KOp::row_of(j), seg_end - 1);
      la.p[j] = reinterpret_cast<const char*>(dy + (size_t)p.ptok[r] * H) + 16 * KOp::chunk_of(j);
    }
    MNOp<WeightRows> lb;
    const char* wbase = reinterpret_cast<const char*>(static_cast<const bf16*>(p.wd) + (size_t)e * H * F + nt * TILE);
    lb.rows = WeightRows{wbase, wbase, (size_t)F * 2, H};
    lb.zero = static_cast<const char*>(p.zeros);
    lb.init(nt * TILE, F);
    int prow[4];   // slot of the wave's row 32i + (lane & 31); its routing weight is loaded after the main loop
#pragma unroll
    for (int i = 0; i < 4; ++i) prow[i] = p.perm[min(r0 + 128 * wm + acc_m(i, lane), seg_end - 1)];
    f32x16 acc[4][2];
    // An expert's last tile often holds a few rows only: each wave multiplies just its 32-row blocks
    // that reach into the segment (none, 1, 2 or all 4), and with at most 128 valid rows the waves
    // 4-7 skip the A loads of rows 128-255. Tiles then differ in cost: the XCD's workgroups take
    // them from a counter.
    const int valid = seg_end - r0 - 128 * wm;   // the wave's rows inside the segment
    const int skip_hi = seg_end - r0 <= 128;
    if (valid <= 0) mainloop<false, true, 32, -1>(acc, smem, la, lb, H / KTILE, 128 * wm, bn, skip_hi);
    else if (valid <= 32) mainloop<false, true, 32, 1>(acc, smem, la, lb, H / KTILE, 128 * wm, bn, skip_hi);
    else if (valid <= 64) mainloop<false, true, 32, 2>(acc, smem, la, lb, H / KTILE, 128 * wm, bn, skip_hi);
    else mainloop<false, true, 32, 0>(acc, smem, la, lb, H / KTILE, 128 * wm, bn, skip_hi);
    fetch();
    float wrow[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) wrow[i] = p.weight[prow[i]];
    // u = dH' staged per 32 rows; each row's 64 columns are read by 8 lanes, 8 columns each. The
    // row pass overwrites u with da and fills a second slab with db (zero on rows or columns past
    // the segment); both then go to the pair-contiguous copy dabT. The wave's partial of g over its
    // 64 columns is partial nt*4 + wn of the row.
    float* slab = wave_slab<2>(smem);
    float* slab2 = slab + NWAVE * Stage<2>::SIZE;
    bf16* __restrict__ dabt = static_cast<bf16*>(p.dabt);
    const int fq = nt * TILE + 64 * wn;
    const int qend = p.qoff[e + 1];
    const int colq = p.qoff[e] + (r0 - p.offsets[e]) + 128 * wm;
    // a/b of the lane's 4 rows of a 32-row block. Row s of block i+1 is loaded into the registers of
    // row s of block i as soon as those are unpacked, so the next block's loads run during the rest
    // of this block (no extra registers). a and b are read once: non-temporal loads, which made
    // this kernel 1.5 % faster.
    uint4 araw[4], braw[4];
    auto load_ab = [&](int i, int s) {
      const int rl = (lane >> 3) + 8 * s, c0 = (lane & 7) * 8;
      const int r = r0 + 128 * wm + 32 * i + rl, f = fq + c0;
      const bf16* abr = ab + (size_t)min(r, seg_end - 1) * 2 * F + min(f, F - 8);
      araw[s] = ld16_nt(abr);
      braw[s] = ld16_nt(abr + F);
    };
#pragma unroll
    for (int s = 0; s < 4; ++s) load_ab(0, s);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      stage_rows(slab, acc, i, lane);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int rl = (lane >> 3) + 8 * s, c0 = (lane & 7) * 8;
        const float wt = __shfl(wrow[i], rl);
        const int r = r0 + 128 * wm + 32 * i + rl, f = fq + c0;
        float gsum = 0.f, da[8], db[8];
        if (r < seg_end && f < F) {
          float u[8], av[8], bv[8];
          read8<2>(slab, rl, c0, u);
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
          bf16* dabr = dab + (size_t)r * 2 * F + f;
          st16_nt(dabr, pack8(da));
          st16_nt(dabr + F, pack8(db));
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) da[e] = db[e] = 0.f;
        }
        if (i < 3) load_ab(i + 1, s);
        constexpr int LD = Stage<2>::LD;
        *reinterpret_cast<float4*>(slab + rl * LD + c0) = make_float4(da[0], da[1], da[2], da[3]);
        *reinterpret_cast<float4*>(slab + rl * LD + c0 + 4) = make_float4(da[4], da[5], da[6], da[7]);
        *reinterpret_cast<float4*>(slab2 + rl * LD + c0) = make_float4(db[0], db[1], db[2], db[3]);
        *reinterpret_cast<float4*>(slab2 + rl * LD + c0 + 4) = make_float4(db[4], db[5], db[6], db[7]);
        gsum = group_sum8(gsum);
        if (r < seg_end && (lane & 7) == 0) p.gpart[(size_t)(nt * 4 + wn) * p.rows + r] = gsum;
      }
      const int colb = colq + 32 * i;
      store_transposed<2>(slab, lane, 64, [&](int c) {
        return colb < qend && fq + c < F ? dabt + (size_t)(fq + c) * p.qc + colb : nullptr;
      });
      store_transposed<2>(slab2, lane, 64, [&](int c) {
        return colb < qend && fq + c < F ? dabt + (size_t)(F + fq + c) * p.qc + colb : nullptr;
      });
    }
  }
}

// the dgrad of h over its M-tile list, from the counter of scheduler slot 0
__device__ __forceinline__ void dh_tiles(const BwdParams& p, char* smem, int* s_tile) {
  TileSched ts(p.sched + 0 * kSchedInts, *p.num_mtiles2 * ((p.F + TILE - 1) / TILE));
  for (int tile = ts.first(s_tile); tile >= 0; tile = ts.next(s_tile)) dh_tile(p, smem, tile, [&] { ts.fetch(); });
}

// the down weight gradient over its XCD's cost-balanced range, round-robin, each tile's first K-tile
// issued before the previous tile's epilogue, which stages its rows as bf16 in ring stage 1 sixteen
// at a time (as the down GEMM).
__device__ __forceinline__ void wgrad_down_tiles(const BwdParams& p, char* smem) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, wm = w >> 1, wn = w & 1;   // 64x128 per wave
  const int H = p.H, F = p.F, ntn = (F + TILE - 1) / TILE, tpe = (H / TILE) * ntn;
  const XcdRange xr = xcd_range_split(p.sched + kSchedWgradDown * kSchedInts);
  MNOp<GatherRows> la;
  KOp lb;
  int e = 0, mt = 0, nt = 0, nk = 0;
  // loaders of tile lid (scalar loads for the tables); B rows hwT[n][qoff[e] ..], contiguous along
  // the expert's pairs (zero-padded to 32)
  auto setup = [&](int lid) {
    e = lid / tpe;
    const int t = lid - e * tpe;
    mt = t / ntn;
    nt = t - mt * ntn;
    const int seg0 = ld_uniform(p.offsets, e), seg_end = ld_uniform(p.offsets, e + 1);
    nk = (seg_end - seg0 + KTILE - 1) / KTILE;
    la.rows = GatherRows{reinterpret_cast<const char*>(static_cast<const bf16*>(p.dy) + mt * TILE), p.ptok,
                         (size_t)H * 2, seg0, seg_end, {}};
    la.zero = static_cast<const char*>(p.zeros);
    la.init(mt * TILE, H);
    const bf16* hwt = static_cast<const bf16*>(p.hwt) + ld_uniform(p.qoff, e);
#pragma unroll
    for (int j = 0; j < LOADS; ++j) {
      const int n = min(nt * TILE + KOp::row_of(j), F - 1);
      lb.p[j] = reinterpret_cast<const char*>(hwt + (size_t)n * p.qc) + 16 * KOp::chunk_of(j);
    }
  };
  const int bn[4] = {128 * wn, 128 * wn + 32, 128 * wn + 64, 128 * wn + 96};
  constexpr int NS = 2 * 32 * 16 / 64;   // epilogue stores per lane of a whole wave block (MI = 2, NJ = 4)
  int lid = xr.first;
  if (lid >= xr.end) return;
  setup(lid);
  if (nk > 0) issue_k0(smem, la, lb);
  bool after_stores = false;
  for (; lid < xr.end; lid += xr.stride) {
    f32x16 acc[2][4];
    mainloop_pre<NS, true, false>(acc, smem, la, lb, nk, 64 * wm, bn, after_stores);
    const int ce = e, cmt = mt, cnt = nt;
    const int mq = cmt * TILE + 64 * wm, nq = cnt * TILE + 128 * wn;
    // every wave is past the main loop's last barrier (or the tile had no K-tile): stage 0 is free
    after_stores = false;
    if (lid + xr.stride < xr.end) {
      setup(lid + xr.stride);
      if (nk > 0) {
        issue_k0(smem, la, lb);
        after_stores = F - nq >= 128;   // the wave's block lies inside F: NS stores follow
      }
    }
    bf16* __restrict__ out = static_cast<bf16*>(p.dwd) + (size_t)ce * H * F;
    store_wave_block_s1<2, 4, 16>(smem, acc, lane, [&](int m) { return out + (size_t)(mq + m) * F + nq; }, F - nq);
  }
}

// backward: [dW_gate; dW_up][e] (2F x H) = sum over the expert's pairs of [da; db]_r x_t^T
__device__ __forceinline__ void wgrad_gateup_tiles(const BwdParams& p, char* smem) {
  // 128x64 per wave: B (x, MN-major) goes through the slower transposing LDS read
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, wm = w >> 2, wn = w & 3;
  const int H = p.H, F = p.F, ntn = H / TILE, tpe = (2 * F / TILE) * ntn;
  const XcdRange xr = xcd_range_split(p.sched + kSchedWgradGateup * kSchedInts);
  const bf16* dabt0 = static_cast<const bf16*>(p.dabt);
  KOp la;
  MNOp<GatherRows> lb;
  int e = 0, mt = 0, nt = 0, nk = 0;
  // loaders of tile lid: A rows dabT[m][qoff[e] ..], contiguous along the expert's pairs (zero-padded
  // to 64); B the expert's gathered x rows
  auto setup = [&](int lid) {
    e = lid / tpe;
    const int t = lid - e * tpe;
    mt = t / ntn;
    nt = t - mt * ntn;
    // scalar loads: after a vector load the compiler would wait for every vector memory operation
    // in flight before using the value
    const int seg0 = ld_uniform(p.offsets, e), seg_end = ld_uniform(p.offsets, e + 1);
    nk = (seg_end - seg0 + KTILE - 1) / KTILE;
    const bf16* dabt = dabt0 + ld_uniform(p.qoff, e);
#pragma unroll
    for (int j = 0; j < LOADS; ++j) {
      const int m = mt * TILE + KOp::row_of(j);
      la.p[j] = reinterpret_cast<const char*>(dabt + (size_t)m * p.qc) + 16 * KOp::chunk_of(j);
    }
    lb.rows = GatherRows{reinterpret_cast<const char*>(static_cast<const bf16*>(p.x) + nt * TILE), p.ptok,
                         (size_t)H * 2, seg0, seg_end, {}};
    lb.zero = static_cast<const char*>(p.zeros);
    lb.init(nt * TILE, H);
  };
  const int bn[2] = {64 * wn, 64 * wn + 32};
  constexpr int NS = 4 * 32 * 8 / 64;   // epilogue stores per lane (MI = 4, NJ = 2)
  int lid = xr.first;
  if (lid >= xr.end) return;
  setup(lid);
  if (nk > 0) issue_k0(smem, la, lb);
  bool after_stores = false;
  for (; lid < xr.end; lid += xr.stride) {
    f32x16 acc[4][2];
    mainloop_pre<NS, false, true>(acc, smem, la, lb, nk, 128 * wm, bn, after_stores);
    const int ce = e, cmt = mt, cnt = nt;
    // every wave is past the main loop's last barrier (or the tile had no K-tile): stage 0 is free
    after_stores = false;
    if (lid + xr.stride < xr.end) {
      setup(lid + xr.stride);
      if (nk > 0) {
        issue_k0(smem, la, lb);
        after_stores = true;
      }
    }
    bf16* __restrict__ dwg = static_cast<bf16*>(p.dwg) + (size_t)ce * F * H;
    bf16* __restrict__ dwu = static_cast<bf16*>(p.dwu) + (size_t)ce * F * H;
    const int mq = cmt * TILE + 128 * wm, nq = cnt * TILE + 64 * wn;
    store_wave_block_s1(smem, acc, lane, [&](int m) {
      const int mm = mq + m;
      return (mm < F ? dwg + (size_t)mm * H : dwu + (size_t)(mm - F) * H) + nq;
    });
  }
}

// backward: dX = [da db] [W_gate[e]; W_up[e]] over a static range per XCD taken round-robin (every
// tile contracts over 2F, so equal counts balance; an expert's half tile does half the MFMAs), each
// tile's first K-tile issued before the previous tile's epilogue, which stages its rows as bf16 in
// ring stage 1 (mainloop_pre_rows).
__device__ __forceinline__ void dgrad_x_tiles_pre(const BwdParams& p, char* smem) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, wm = w >> 2, wn = w & 3;   // 128x64 per wave
  const int H = p.H, F = p.F, ntn = H / TILE, nk = 2 * F / KTILE;
  const XcdRange xr = xcd_range(ld_uniform(p.num_mtiles2, 0) * ntn);
  const bf16* __restrict__ dab = static_cast<const bf16*>(p.dab);
  bf16* __restrict__ dxp = static_cast<bf16*>(p.dxp);
  KOp la;
  MNOp<WeightRows> lb;
  int r0 = 0, seg_end = 0, nt = 0;
  bool half = false;
  // loaders of tile `tile`; scalar loads for the tables (a vector load's compiler-inserted wait
  // would also wait for the direct-to-LDS loads in flight)
  auto setup = [&](int tile) {
    const int mt = tile / ntn;
    nt = tile - mt * ntn;
    const int e = ld_uniform(reinterpret_cast<const int*>(p.mtile2), 2 * mt);
    r0 = ld_uniform(reinterpret_cast<const int*>(p.mtile2), 2 * mt + 1);
    seg_end = ld_uniform(p.offsets, e + 1);
    half = seg_end - r0 <= 128;
#pragma unroll
    for (int j = 0; j < LOADS; ++j) {
      const int r = min(r0 + KOp::row_of(j), seg_end - 1);
      la.p[j] = reinterpret_cast<const char*>(dab + (size_t)r * 2 * F) + 16 * KOp::chunk_of(j);
    }
    lb.rows = WeightRows{reinterpret_cast<const char*>(static_cast<const bf16*>(p.wg) + (size_t)e * F * H + nt * TILE),
                         reinterpret_cast<const char*>(static_cast<const bf16*>(p.wu) + (size_t)e * F * H + nt * TILE),
                         (size_t)H * 2, F};
    lb.zero = static_cast<const char*>(p.zeros);
    lb.init(nt * TILE, H);
  };
  const int bn[2] = {64 * wn, 64 * wn + 32};
  constexpr int NS = 4 * 32 * 8 / 64;   // epilogue stores per lane of a full tile (MI = 4, NJ = 2)
  int lid = xr.first;
  if (lid >= xr.end) return;
  setup(lid);
  issue_k0(smem, la, lb, half && wave_id() >= NWAVE / 2);
  bool after_stores = false;
  for (; lid < xr.end; lid += xr.stride) {
    f32x16 acc[4][2];
    mainloop_pre_rows<NS, false, true, 64>(acc, smem, la, lb, nk, 32 * wm, bn, after_stores, half);
    const int cr0 = r0, cseg = seg_end, cnt = nt;
    // every wave is past the main loop's last barrier: stage 0 is free
    after_stores = false;
    if (lid + xr.stride < xr.end) {
      setup(lid + xr.stride);
      issue_k0(smem, la, lb, half && wave_id() >= NWAVE / 2);
      after_stores = cseg - cr0 >= TILE;   // every row of the tile is stored: NS stores follow
    }
    const int rq = cr0 + 32 * wm;   // the wave's row m is tile row 32 wm + 64 (m / 32) + m % 32
    bf16* const oq = dxp + cnt * TILE + 64 * wn;
    store_wave_block_s1(smem, acc, lane, [&](int m) {
      const int r = rq + 64 * (m >> 5) + (m & 31);
      return r < cseg ? oq + (size_t)r * H : nullptr;
    });
  }
}

// The backward GEMMs as kernels. On an expert share too (16 of 128 experts of the 30B-A3B layer:
// about 16 k pairs, 204 dH tiles for 256 CUs) they fill each other's tails on the two streams: 3 %
// faster there than two launches of two GEMMs each from one tile queue per XCD.
__global__ __launch_bounds__(NTHR8, 1) void k_bwd_dh_bf16(BwdParams p) {
  MOE_SMEM
  __shared__ int s_tile;
  dh_tiles(p, smem, &s_tile);
}
__global__ __launch_bounds__(NTHR8, 1) void k_dgrad_x_bf16(BwdParams p) {
  MOE_SMEM
  dgrad_x_tiles_pre(p, smem);
}
__global__ __launch_bounds__(NTHR8, 1) void k_wgrad_down_bf16(BwdParams p) {
  MOE_SMEM
  wgrad_down_tiles(p, smem);
}
__global__ __launch_bounds__(NTHR8, 1) void k_wgrad_gateup_bf16(BwdParams p) {
  MOE_SMEM
  wgrad_gateup_tiles(p, smem);
}

// ------------------------------------------------------------------------------------------------
// Router projection in front of the layer: logits = x W_r^T (fp32), and in the backward
// dW_r = dlogits^T x and dx += dlogits W_r. The pages fold the routing into the fused call ("Prime
// Mega MoE: kernel fuso per l'addestramento MoE" on "Prime Mega MoE: il kernel che accelera il
// training AI del 55%"); the projection is read as the usual linear router without bias. E is small
// (128 at the benchmark shape), so the two GEMMs with a long contraction (over H in the forward,
// over T for dW_r) split it p.S ways and add the fp32 partial sums in a fixed order afterwards: no
// atomics, so results stay bitwise reproducible. The backward multiplies a bf16 copy of dlogits.

// contraction rows k0 .. kend-1 of a row-major matrix (row k at base + k*ld); rows at or past kend
// read the zero page
struct DenseRows {
  const char* base;
  size_t ld;
  int k0, kend;
  __device__ __forceinline__ void prefetch(int) {}
  __device__ __forceinline__ void prologue_prefetch(int) {}
  __device__ __forceinline__ const char* row(int kt, int j) const {
    const int k = k0 + kt * KTILE + mn_krow(j);
    return k < kend ? base + (size_t)k * ld : nullptr;
  }
  __device__ __forceinline__ const char* prologue_row(int kt, int j) const { return row(kt, j); }
};

// Stores the wave's block as fp32: out_row(m) is the output row of the wave's row m at its first
// column, or null to skip the row; ncols limits the columns (in steps of 8).
template <int MI, int NJ, class OutRow>
__device__ __forceinline__ void store_block_f32(char* smem, const f32x16 (&acc)[MI][NJ], int lane, OutRow out_row,
                                                int ncols) {
  constexpr int LPR = 4 * NJ, RPP = 64 / LPR;
  float* slab = wave_slab<NJ>(smem);
#pragma unroll
  for (int i = 0; i < MI; ++i) {
    stage_rows(slab, acc, i, lane);
#pragma unroll
    for (int s = 0; s < 32 / RPP; ++s) {
      const int rl = lane / LPR + RPP * s, c0 = (lane % LPR) * 8;
      float* o = out_row(32 * i + rl);
      if (o && c0 < ncols) {
        float v[8];
        read8<NJ>(slab, rl, c0, v);
        st16(o + c0, make_uint4(__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]),
                                __float_as_uint(v[3])));
        st16(o + c0 + 4, make_uint4(__float_as_uint(v[4]), __float_as_uint(v[5]), __float_as_uint(v[6]),
                                    __float_as_uint(v[7])));
      }
    }
  }
}

// Adds the wave's block to bf16 rows (read, add in fp32, round once, write); out_row as above, all
// 32 NJ columns.
template <int MI, int NJ, class OutRow>
__device__ __forceinline__ void add_block_bf16(char* smem, const f32x16 (&acc)[MI][NJ], int lane, OutRow out_row) {
  constexpr int LPR = 4 * NJ, RPP = 64 / LPR;
  float* slab = wave_slab<NJ>(smem);
#pragma unroll
  for (int i = 0; i < MI; ++i) {
    stage_rows(slab, acc, i, lane);
#pragma unroll
    for (int s = 0; s < 32 / RPP; ++s) {
      const int rl = lane / LPR + RPP * s, c0 = (lane % LPR) * 8;
      bf16* o = out_row(32 * i + rl);
      if (o) {
        float v[8], u[8];
        read8<NJ>(slab, rl, c0, v);
        unpack8(ld16(o + c0), u);
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] += u[e];
        st16(o + c0, pack8(v));
      }
    }
  }
}

// forward: part[s][t][e] = sum over the s-th kc-element slice of H of x[t][h] W_r[e][h]
__global__ __launch_bounds__(NTHR8, 1) void k_router_fwd_bf16(RouterParams p) {
  MOE_SMEM
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, wm = w >> 1, wn = w & 1;   // 64x128 per wave
  const bf16* __restrict__ x = static_cast<const bf16*>(p.x);
  const bf16* __restrict__ wr = static_cast<const bf16*>(p.wr);
  const int T = (int)p.T, H = p.H, E = p.E, Ep = p.Ep;
  const int mtn = (T + TILE - 1) / TILE, ntn = (E + TILE - 1) / TILE, per = mtn * ntn;
  const XcdRange xr = xcd_range(per * p.S);
  const int bn[4] = {128 * wn, 128 * wn + 32, 128 * wn + 64, 128 * wn + 96};
  for (int tile = xr.first; tile < xr.end; tile += xr.stride) {
    const int sp = tile / per, t = tile - sp * per, mt = t / ntn, nt = t - mt * ntn;
    KOp la, lb;
#pragma unroll
    for (int j = 0; j < LOADS; ++j) {
      const int row = KOp::row_of(j), c = KOp::chunk_of(j);
      const size_t k0 = (size_t)sp * p.kc;
      la.p[j] = reinterpret_cast<const char*>(x + (size_t)min(mt * TILE + row, T - 1) * H + k0) + 16 * c;
      lb.p[j] = reinterpret_cast<const char*>(wr + (size_t)min(nt * TILE + row, E - 1) * H + k0) + 16 * c;
    }
    f32x16 acc[2][4];
    mainloop<false, false>(acc, smem, la, lb, p.kc / KTILE, 64 * wm, bn);
    float* out = p.part + (size_t)sp * T * Ep;
    const int m0 = mt * TILE + 64 * wm, n0 = nt * TILE + 128 * wn;
    store_block_f32(smem, acc, lane, [&](int m) { return m0 + m < T ? out + (size_t)(m0 + m) * Ep + n0 : nullptr; },
                    Ep - n0);
  }
}

// forward: logits[t][e] = sum over s (S <= 4), in order, of part[s][t][e]; 4 columns of the padded rows per
// thread (the loads of all slices are issued before the adds)
__global__ __launch_bounds__(256) void k_router_sum_logits(RouterParams p) {
  const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t nq = p.T * (p.Ep / 4);
  if (q >= nq) return;
  const int64_t t = q / (p.Ep / 4), e = (q - t * (p.Ep / 4)) * 4;
  float4 v[4];
#pragma unroll
  for (int s = 0; s < 4; ++s)
    v[s] = s < p.S ? *reinterpret_cast<const float4*>(p.part + ((size_t)s * p.T + t) * p.Ep + e) : make_float4(0.f, 0.f, 0.f, 0.f);
  float r[4] = {v[0].x, v[0].y, v[0].z, v[0].w};
#pragma unroll
  for (int s = 1; s < 4; ++s) {
    r[0] += v[s].x; r[1] += v[s].y; r[2] += v[s].z; r[3] += v[s].w;
  }
  float* out = p.logits + t * p.E;
#pragma unroll
  for (int c = 0; c < 4; ++c)
    if (e + c < p.E) out[e + c] = r[c];
}

// backward: dlb = bf16(dlogits), zero-padded to Ep columns (8 per thread: Ep is a multiple of 64, so
// a thread's 8 stay in one row; 16-byte loads when dlogits and its rows are 16-byte aligned); the
// zero page
__global__ __launch_bounds__(256) void k_router_dl_bf16(RouterParams p) {
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8;
  if (blockIdx.x == 0 && threadIdx.x < kZeroBytes / 16) static_cast<uint4*>(p.zeros)[threadIdx.x] = make_uint4(0u, 0u, 0u, 0u);
  if (i >= p.T * p.Ep) return;
  const int64_t t = i / p.Ep;
  const int c = (int)(i - t * p.Ep);
  const float* src = p.dlogits + t * p.E + c;
  float v[8];
  if ((p.E & 3) == 0 && (reinterpret_cast<uintptr_t>(p.dlogits) & 15) == 0 && c + 8 <= p.E) {
    const float4 a = *reinterpret_cast<const float4*>(src), b = *reinterpret_cast<const float4*>(src + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = c + e < p.E ? src[e] : 0.f;
  }
  *reinterpret_cast<uint4*>(static_cast<bf16*>(p.dlb) + i) = pack8(v);
}

// backward: dx[t][h] += sum_e dlb[t][e] W_r[e][h] (contraction over E; W_r is MN-major here)
__global__ __launch_bounds__(NTHR8, 1) void k_router_dx_bf16(RouterParams p) {
  MOE_SMEM
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, wm = w >> 1, wn = w & 1;   // 64x128 per wave
  const bf16* __restrict__ dlb = static_cast<const bf16*>(p.dlb);
  bf16* __restrict__ dx = static_cast<bf16*>(p.dx);
  const int T = (int)p.T, H = p.H, Ep = p.Ep;
  const int mtn = (T + TILE - 1) / TILE, ntn = H / TILE;
  const XcdRange xr = xcd_range(mtn * ntn);
  const int bn[4] = {128 * wn, 128 * wn + 32, 128 * wn + 64, 128 * wn + 96};
  for (int tile = xr.first; tile < xr.end; tile += xr.stride) {
    const int mt = tile / ntn, nt = tile - mt * ntn;
    KOp la;
#pragma unroll
    for (int j = 0; j < LOADS; ++j)
      la.p[j] = reinterpret_cast<const char*>(dlb + (size_t)min(mt * TILE + KOp::row_of(j), T - 1) * Ep) +
                16 * KOp::chunk_of(j);
    MNOp<DenseRows> lb;
    lb.rows = DenseRows{reinterpret_cast<const char*>(static_cast<const bf16*>(p.wr) + nt * TILE), (size_t)H * 2, 0, p.E};
    lb.zero = static_cast<const char*>(p.zeros);
    lb.init(nt * TILE, H);
    f32x16 acc[2][4];
    mainloop<false, true>(acc, smem, la, lb, Ep / KTILE, 64 * wm, bn);
    const int m0 = mt * TILE + 64 * wm;
    bf16* const oq = dx + nt * TILE + 128 * wn;
    add_block_bf16(smem, acc, lane, [&](int m) { return m0 + m < T ? oq + (size_t)(m0 + m) * H : nullptr; });
  }
}

// backward: part[s][e][h] = sum over the s-th kc-token slice of dlb[t][e] x[t][h] (both operands
// MN-major: the contraction runs over the tokens)
__global__ __launch_bounds__(NTHR8, 1) void k_router_dw_bf16(RouterParams p) {
  MOE_SMEM
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, wm = w >> 1, wn = w & 1;   // 64x128 per wave
  const int T = (int)p.T, H = p.H, E = p.E, Ep = p.Ep;
  const int mtn = (E + TILE - 1) / TILE, ntn = H / TILE, per = mtn * ntn;
  const XcdRange xr = xcd_range(per * p.S);
  const int bn[4] = {128 * wn, 128 * wn + 32, 128 * wn + 64, 128 * wn + 96};
  for (int tile = xr.first; tile < xr.end; tile += xr.stride) {
    const int sp = tile / per, t = tile - sp * per, mt = t / ntn, nt = t - mt * ntn;
    const int k0 = sp * p.kc, kend = min(T, k0 + p.kc);
    MNOp<DenseRows> la, lb;
    la.rows = DenseRows{reinterpret_cast<const char*>(static_cast<const bf16*>(p.dlb) + mt * TILE), (size_t)Ep * 2, k0, kend};
    la.zero = static_cast<const char*>(p.zeros);
    la.init(mt * TILE, Ep);
    lb.rows = DenseRows{reinterpret_cast<const char*>(static_cast<const bf16*>(p.x) + nt * TILE), (size_t)H * 2, k0, kend};
    lb.zero = la.zero;
    lb.init(nt * TILE, H);
    f32x16 acc[2][4];
    mainloop<true, true>(acc, smem, la, lb, (kend - k0 + KTILE - 1) / KTILE, 64 * wm, bn);
    float* out = p.part + (size_t)sp * E * H;
    const int m0 = mt * TILE + 64 * wm, n0 = nt * TILE + 128 * wn;
    store_block_f32(smem, acc, lane, [&](int m) { return m0 + m < E ? out + (size_t)(m0 + m) * H + n0 : nullptr; }, 128);
  }
}

// backward: dW_r[e][h] = bf16(sum over s, in order, of part[s][e][h]); 4 elements per thread, the
// slices' loads issued 8 at a time ahead of their adds
__global__ __launch_bounds__(256) void k_router_sum_dw(RouterParams p) {
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  const int64_t n = (int64_t)p.E * p.H;
  if (i >= n) return;
  float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s0 = 0; s0 < p.S; s0 += 8) {
    float4 q[8];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      q[u] = s0 + u < p.S ? *reinterpret_cast<const float4*>(p.part + (size_t)(s0 + u) * n + i) : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      v.x += q[u].x; v.y += q[u].y; v.z += q[u].z; v.w += q[u].w;
    }
  }
  st8(static_cast<bf16*>(p.dwr) + i, pack4(v.x, v.y, v.z, v.w));
}

// One workgroup before the backward GEMMs: zeroes the tile-scheduler counters (the workspace is the
// caller's) and cuts each weight-gradient GEMM's tile list (expert-major, tpe tiles per expert) into
// 8 contiguous per-XCD ranges, whose tiles the XCD's workgroups then take round-robin. Every tile of
// expert e contracts over the expert's c_e pairs: u_e = ceil(c_e / ktile) K-tiles, plus
// kTileOverhead K-tiles' worth of prologue and epilogue. Ranges of equal tile count are kept while
// their estimated costs stay within 10 % of each other (then every workgroup also gets the same
// number of tiles); otherwise, as under a skewed load, where equal counts gave the XCD holding the
// most loaded experts several times the others' work, boundary x (1..7) moves to the first tile whose
// preceding tiles cost at least x/8 of the total. El <= kMaxExperts = 512: 2 experts per thread.
constexpr int kTileOverhead = 2;
__global__ __launch_bounds__(256) void k_sched_setup(int* sched, const int* offsets, int El, int tpe_d, int tpe_g,
                                                     int ktile) {
  __shared__ long long part[256];   // inclusive prefix of the per-thread cost sums
  __shared__ int uu[2 * 256];       // u_e
  __shared__ int even[2];           // equal-count ranges within 10 %
  const int t = threadIdx.x;
  for (int i = t; i < kSchedSlots * kSchedInts; i += 256) sched[i] = 0;
  long long own = 0;
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int e = 2 * t + q;
    const int u = e < El ? (offsets[e + 1] - offsets[e] + ktile - 1) / ktile + kTileOverhead : 0;
    uu[e] = u;
    own += u;
  }
  part[t] = own;
  __syncthreads();
  for (int d = 1; d < 256; d <<= 1) {
    const long long v = t >= d ? part[t - d] : 0;
    __syncthreads();
    part[t] += v;
    __syncthreads();
  }
  const long long total = part[255];
  const int slots[2] = {kSchedWgradDown, kSchedWgradGateup}, tpes[2] = {tpe_d, tpe_g};
  // cost of tiles [0, L): the experts before e = L / tpe, then L % tpe tiles of e
  auto cum = [&](int tpe, int L) -> long long {
    const int e = L / tpe, j = L - e * tpe;
    long long U = e >= 2 ? part[e / 2 - 1] : 0;
    if (e & 1) U += uu[e - 1];
    return tpe * U + (e < El ? (long long)j * uu[e] : 0);
  };
  if (t < 2) {
    const int tpe = tpes[t], per = (El * tpe + 7) >> 3;
    long long mx = 0;
    for (int x = 0; x < 8; ++x)
      mx = max(mx, cum(tpe, min((x + 1) * per, El * tpe)) - cum(tpe, min(x * per, El * tpe)));
    even[t] = 10 * 8 * mx <= 11 * tpe * total;
  }
  __syncthreads();
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    const int tpe = tpes[g], per = (El * tpe + 7) >> 3;
    int* b = sched + slots[g] * kSchedInts;
    if (even[g]) {
      if (t < 8) b[t + 1] = min((t + 1) * per, El * tpe);
      continue;
    }
    long long pre = part[t] - own;      // cost units of the experts before 2t
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int e = 2 * t + q;
      if (e < El) {
        const long long u = uu[e], lo = tpe * pre, hi = tpe * (pre + u);
        for (int x = 1; x < 8; ++x) {
          const long long target = tpe * total * x / 8;
          if (lo <= target && target < hi) b[x] = e * tpe + (int)((target - lo + u - 1) / u);
        }
        pre += u;
      }
    }
    if (t == 0) b[8] = El * tpe;
  }
}

// zeroes the kSchedSlots tile-scheduler slots at sched (a kernel rather than a memset: the call may be
// captured in a graph)
__global__ __launch_bounds__(256) void k_zero_sched(int* sched) {
  for (int i = threadIdx.x; i < kSchedSlots * kSchedInts; i += 256) sched[i] = 0;
}

}  // namespace

hipError_t launch_sched_setup(const BwdParams& p, int ktile, hipStream_t s) {
  const int tpe_d = (p.H / TILE) * ((p.F + TILE - 1) / TILE), tpe_g = (2 * p.F / TILE) * (p.H / TILE);
  prof_mark_begin("sched_setup", s);
  k_sched_setup<<<1, 256, 0, s>>>(p.sched, p.offsets, p.El, tpe_d, tpe_g, ktile);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  prof_mark_end(s);
  return hipSuccess;
}

hipError_t launch_forward_gemms_bf16(const FwdParams& p, int grid, hipStream_t s, bool recompute) {
  hipError_t err;
  if (recompute) {   // the backward's recompute: its own tile counters, zeroed here
    k_zero_sched<<<1, 256, 0, s>>>(p.sched);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  prof_mark_begin(recompute ? "gemm_gateup_recompute" : "gemm_gateup_swiglu", s);
  if (p.hwtq) k_gateup_bf16<true><<<grid, NTHR8, 0, s>>>(p);
  else k_gateup_bf16<false><<<grid, NTHR8, 0, s>>>(p);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  prof_mark_end(s);
  if (recompute) return hipSuccess;
  prof_mark_begin("gemm_down", s);
  k_down_bf16<<<grid, NTHR8, 0, s>>>(p);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  prof_mark_end(s);
  return hipSuccess;
}

hipError_t launch_router_fwd_bf16(const RouterParams& p, int grid, hipStream_t s) {
  hipError_t err;
  prof_mark_begin("router_fwd_gemm", s);
  k_router_fwd_bf16<<<grid, NTHR8, 0, s>>>(p);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  prof_mark_end(s);
  prof_mark_begin("router_fwd_sum", s);
  k_router_sum_logits<<<(unsigned)((p.T * (p.Ep / 4) + 255) / 256), 256, 0, s>>>(p);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  prof_mark_end(s);
  return hipSuccess;
}

hipError_t launch_router_bwd_bf16(const RouterParams& p, int grid, hipStream_t s) {
  hipError_t err;
  prof_mark_begin("router_dlogits_bf16", s);
  k_router_dl_bf16<<<(unsigned)((p.T * p.Ep / 8 + 255) / 256), 256, 0, s>>>(p);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  prof_mark_end(s);
  prof_mark_begin("router_dx_gemm", s);
  k_router_dx_bf16<<<grid, NTHR8, 0, s>>>(p);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  prof_mark_end(s);
  prof_mark_begin("router_dw_gemm", s);
  k_router_dw_bf16<<<grid, NTHR8, 0, s>>>(p);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  prof_mark_end(s);
  prof_mark_begin("router_dw_sum", s);
  k_router_sum_dw<<<(unsigned)(((int64_t)p.E * p.H / 4 + 255) / 256), 256, 0, s>>>(p);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  prof_mark_end(s);
  return hipSuccess;
}

// dH, then the dgrad of x, on the caller's stream (the critical path to the dx combine); the two
// weight gradients on the device's side stream when there is one (on s otherwise), the down one from
// the start (it needs only dY and w h), the gate/up one after dH. Their workgroups take the CUs that
// dH's and the dgrad's free in those kernels' tails; the caller's stream waits for them after the dx
// combine (side_stream_join).
hipError_t launch_backward_gemms_bf16(const BwdParams& p, int grid, hipStream_t s) {
  hipError_t err;
  if ((err = launch_sched_setup(p, KTILE, s)) != hipSuccess) return err;
  hipStream_t s1 = side_stream_fork(s);
  hipStream_t sw = s1 ? s1 : s;   // the weight gradients' stream
  prof_mark_begin("gemm_bwd_dh_dswiglu", s);
  k_bwd_dh_bf16<<<grid, NTHR8, 0, s>>>(p);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  prof_mark_end(s);
  if (s1 && (err = side_stream_mark(s)) != hipSuccess) return err;   // dH done: the gate/up one may start
  prof_mark_begin("gemm_wgrad_down", sw);
  k_wgrad_down_bf16<<<grid, NTHR8, 0, sw>>>(p);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  prof_mark_end(sw);
  if (s1 && (err = side_stream_wait_mark()) != hipSuccess) return err;
  prof_mark_begin("gemm_dgrad_x", s);
  k_dgrad_x_bf16<<<grid, NTHR8, 0, s>>>(p);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  prof_mark_end(s);
  prof_mark_begin("gemm_wgrad_gateup", sw);
  k_wgrad_gateup_bf16<<<grid, NTHR8, 0, sw>>>(p);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  prof_mark_end(sw);
  return hipSuccess;
}

}  // namespace moe
