/*
 * moe.h - C ABI of libmoe.so, a fused Mixture-of-Experts layer (forward and backward) for one
 * AMD Instinct MI355X (gfx950).
 *
 * What the layer computes. The pages on Prime Intellect's "Prime Mega MoE" (an extension of
 * DeepSeek's "Mega MoE") describe one fused call per pass:
 *  - "A Magia da Fusão" on "IA: MoE Kernel 3x Mais Rápido Chegou!" lists its steps: dispatch of
 *    tokens to experts, the experts' linear layers, SwiGLU, and the combine of the results.
 *  - "Afinal, o que é esse Prime Mega MoE?" on the same page adds the backward pass.
 *  - "Detalhes Técnicos Rápidos" on the same page requires gated SwiGLU experts without biases,
 *    hidden size a multiple of 256 and expert FFN size a multiple of 128.
 *  - "Supporto di precisione e vincoli hardware" on "Prime Mega MoE: il kernel che accelera il
 *    training AI del 55%" gives the precision modes.
 *
 * With T tokens, hidden size H, expert FFN size F, E routed experts and top-k routing:
 *    S_t  = the k largest router logits of token t (ties to the lower expert index)
 *    w_tj = exp(l_{t,S_tj}) / sum_i exp(l_{t,S_ti})        (softmax renormalised over S_t)
 *    y_t  = sum_j w_tj * W_down[e] (silu(W_gate[e] x_t) * (W_up[e] x_t)),  e = S_tj
 * The backward returns dx, dlogits (through the renormalised softmax) and dW_gate, dW_up,
 * dW_down for the gradient dy of y.
 *
 * Expert share. The library computes the experts [expert_offset, expert_offset + E_local) of
 * E_total. Routing always runs over all E_total experts, and w stays renormalised over the
 * full top-k. Pairs routed outside the share are skipped. Outputs y, dx and dlogits are then
 * this share's linear contribution: summed over all shares they give the full layer.
 *
 * Conventions common to every entry point:
 *  - Every pointer is a device pointer unless the comment says "host". The caller allocates
 *    every buffer, including the workspace and the saved-activation buffer sized by
 *    moe_query_sizes(). The library never allocates, frees or caches device memory.
 *  - All tensors are dense row-major. Let elem be float in MOE_MODE_FP32 and bf16 (raw 16-bit
 *    storage) in every other mode:
 *      x, y, dy, dx                  [T, H]            elem
 *      logits, dlogits               [T, E_total]      float (fp32)
 *      w_gate, w_up, dw_gate, dw_up  [E_local, F, H]   elem (out x in, K contiguous)
 *      w_down, dw_down               [E_local, H, F]   elem
 *  - stream is a hipStream_t (NULL: the default stream) of the calling thread's current device,
 *    where every buffer lives (another device's stream: MOE_ERR_INVALID_ARG). Every call only
 *    enqueues work on it and returns. No call synchronises the host or copies device data to the
 *    host.
 *  - Validation happens on the host before anything is enqueued. On any error nothing is
 *    enqueued and no output is touched. Launch failures return MOE_ERR_HIP. A device fault
 *    surfaces at the caller's next synchronisation.
 *  - Preconditions that are not checked: logits are finite, and buffers do not overlap.
 *  - Results are deterministic: no floating-point atomics anywhere, so repeated calls give
 *    bitwise-identical outputs.
 *  - The library keeps no state between calls apart from the profiling records, a
 *    thread-local error string and, per device, one more stream with three events, which the
 *    first moe_bwd on that device outside graph capture creates (at default priority). moe_bwd
 *    runs its two weight-gradient GEMMs there: that stream first waits for everything enqueued
 *    on `stream` before the call, and `stream` waits for it before any work enqueued after the
 *    call, so the ordering seen on `stream` is as if all ran there. moe_bwd calls on one device
 *    share that stream. Calls on different streams may run concurrently if their buffers are
 *    distinct.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Precision modes ("Supporto di precisione e vincoli hardware"; "A Magia da Fusão"):
 *   FP32     all storage and arithmetic in fp32 (test mode).
 *   BF16     bf16 storage; GEMMs on bf16 MFMA with fp32 accumulation; routing,
 *            softmax, SwiGLU and combines in fp32.
 *   MXFP8    bf16 storage; every GEMM operand quantised to MXFP8 in both passes, GEMMs on
 *            the scaled fp8 MFMA with fp32 accumulation. The format is read as OCP
 *            microscaling: one e8m0 scale 2^s per 32 consecutive elements along the GEMM's
 *            contraction axis, s = floor(log2 amax) - 8 clamped to [-127, 127], elements e4m3
 *            (finite-only, largest 448) of v / 2^s, rounded to nearest even and saturated.
 *            Quantised operands (contraction axis in brackets):
 *              forward   x, W_gate, W_up [H]; w*h, W_down [F]
 *              backward  dy, W_down [H]; da, db, W_gate, W_up [F];
 *                        dy, w*h, da, db, x [the expert's pairs in sorted order, blocks of 32
 *                        from the expert's first pair, the last block zero-padded]
 *            Routing, softmax, SwiGLU, the router gradient and the combines stay fp32.
 *   FP8_BWD  the BF16 forward; the backward GEMMs quantised as in MXFP8.
 *   FP8      blockwise-scaled FP8 in both passes (the pages list it without block sizes). The
 *            same operands and axes as MXFP8, on the same scaled fp8 MFMA, with larger blocks and
 *            a scale that never saturates:
 *              activation operands (x, dy, w*h, da, db): one scale per 128 consecutive elements
 *                along the contraction axis (for the weight gradients, 128 pairs from the expert's
 *                first pair, the last block zero-padded);
 *              weights: one scale per 128 x 128 tile of each expert's matrix, the same for both
 *                orientations;
 *              scale 2^s with s the smallest integer such that amax <= 448 * 2^s, clamped to
 *                [-127, 127] (-127 for an all-zero block); elements e4m3 of v / 2^s, rounded to
 *                nearest even. */
typedef enum {
  MOE_MODE_FP32 = 0,
  MOE_MODE_BF16 = 1,
  MOE_MODE_MXFP8 = 2,
  MOE_MODE_FP8_BWD = 3,
  MOE_MODE_FP8 = 4
} moe_mode;

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1,        /* null pointer, non-positive size, k > E_total, bad share,
                                     recompute not 0 or 1 */
  MOE_ERR_UNSUPPORTED_SHAPE = 2,  /* H % 256, F % 128, E_total > 512, k > 32, T*k >= 2^31 */
  MOE_ERR_UNSUPPORTED_MODE = 3,   /* mode value unknown */
  MOE_ERR_WORKSPACE_TOO_SMALL = 4,
  MOE_ERR_HIP = 5                 /* a HIP runtime call failed; see moe_last_error() */
} moe_status;

/* Layer description; passed by host pointer to every call. */
typedef struct {
  int64_t T;              /* tokens, >= 1 */
  int32_t H;              /* hidden size, multiple of 256 */
  int32_t F;              /* expert FFN size, multiple of 128 */
  int32_t E_total;        /* routed experts, 1..512 */
  int32_t E_local;        /* experts computed here, >= 1 */
  int32_t expert_offset;  /* first computed expert; expert_offset + E_local <= E_total */
  int32_t topk;           /* experts per token, 1..min(E_total, 32) */
  int32_t mode;           /* moe_mode */
  int32_t recompute;      /* 0 or 1: activation checkpointing (see below) */
} moe_desc;

/* Activation checkpointing (desc.recompute). The pages quote the layer's cost under full
 * activation checkpointing as two forwards plus one backward ("Analisi dei kernel layer: forward vs
 * backward" and "Benchmark di training end-to-end: velocità o illusione?" on "Prime Mega MoE: il
 * kernel che accelera il training AI del 55%"): the training step runs the forward once, keeps only
 * its input, and runs it again inside the backward.
 *   recompute = 0  moe_fwd leaves the gate/up activations (a, b and w*h; in MXFP8 and FP8 also the
 *                  weights quantised for the backward) in `saved`, and moe_bwd reads them.
 *   recompute = 1  moe_fwd keeps only the routing results in `saved` and writes no activation for
 *                  the backward. moe_bwd first recomputes a, b and w*h (and, in the fp8 modes, the
 *                  quantised x and weights) from x with the forward's own gate/up kernel, into its
 *                  workspace, then runs the backward. Only the gate/up GEMM is recomputed: the down
 *                  GEMM and the combine do not feed the backward.
 * The recomputed values are the same bits as the forward's (same kernels, same inputs), so every
 * output of moe_bwd is bitwise identical to recompute = 0. moe_query_sizes gives the smaller
 * `saved` and the larger backward workspace of the chosen form. */

/* Byte sizes of the caller-allocated buffers for the description (host pointers out; any may
 * be NULL). Each size is a multiple of 256. The base pointers must be 256-byte aligned.
 *   fwd_ws   workspace for moe_route and moe_fwd (contents need not be preserved)
 *   bwd_ws   workspace for moe_bwd
 *   saved    routing metadata and activations written by moe_fwd/moe_route and read by
 *            moe_bwd; it must stay untouched between the two calls.
 * Host-only: no device work. */
moe_status moe_query_sizes(const moe_desc* d, size_t* fwd_ws, size_t* bwd_ws, size_t* saved);

/* Routing only ("A Magia da Fusão": dispatch; "kernel fuso per l'addestramento MoE": routing
 * is part of the fused operation). Writes the routing half of `saved` (layout below).
 * moe_fwd does this itself; this entry point exists so that routing can be tested alone. */
moe_status moe_route(const moe_desc* d, const float* logits, void* saved, void* ws,
                     size_t ws_bytes, void* stream);

/* moe_route without a workspace, for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation). Same results in `saved` as
 * moe_route. The routing scratch (per 64 tokens and local expert 16 bytes of token masks, counts and
 * prefixes, plus 512 bytes of tile counters) lives in a static device array of 8 MiB inside the
 * library, one per GPU, held until the process ends; a description needing more returns
 * MOE_ERR_UNSUPPORTED_SHAPE (up to 262,080 tokens at 128 local experts). Nothing is allocated or
 * freed. Every call on one GPU shares that GPU's array: calls that overlap on one GPU (different
 * streams, or host threads) race, and must be ordered by the caller. The first call on a device
 * looks up the array's address there (a host-side runtime query, no device work). */
moe_status moe_route_static(const moe_desc* d, const float* logits, void* saved, void* stream);

/* Forward: routing, dispatch (gathered inside the gate/up GEMM's operand loads), gate/up GEMM
 * with the SwiGLU epilogue, down GEMM, and the weighted combine into y. y is overwritten.
 * `saved` receives what moe_bwd needs. */
moe_status moe_fwd(const moe_desc* d, const void* x, const float* logits,
                   const void* w_gate, const void* w_up, const void* w_down,
                   void* y, void* saved, void* ws, size_t ws_bytes, void* stream);

/* The forward from x: the router projection logits = x w_router^T fused with the routing (top-k,
 * weights and the per-block expert masks in one kernel), then the layer as moe_fwd. The pages fold the
 * routing into the fused operation ("Prime Mega MoE: kernel fuso per l'addestramento MoE" on "Prime
 * Mega MoE: il kernel che accelera il training AI del 55%"); the projection is the linear router of
 * moe_router_fwd. `logits` [T, E_total] fp32 is an output here: the logits the routing used, so
 * that the routing is exactly oracle routing of `logits` (moe_router_fwd runs the same projection
 * kernel, so moe_router_fwd then moe_fwd routes alike). w_router [E_total, H] bf16, 16-byte aligned.
 * The backward is moe_bwd, then moe_router_bwd with moe_bwd's dlogits.
 * Bf16 I/O modes only (MOE_ERR_UNSUPPORTED_MODE in MOE_MODE_FP32), E_total <= 256 and topk <= 8
 * (MOE_ERR_UNSUPPORTED_SHAPE otherwise: use moe_router_fwd, then moe_fwd). Workspace and `saved` as
 * for moe_fwd. */
moe_status moe_fwd_router(const moe_desc* d, const void* x, const void* w_router, float* logits,
                          const void* w_gate, const void* w_up, const void* w_down, void* y,
                          void* saved, void* ws, size_t ws_bytes, void* stream);

/* Backward of <dy, y> with the same x, weights and the `saved` of the matching moe_fwd (in
 * MOE_MODE_MXFP8 and MOE_MODE_FP8 without recompute, `saved` also carries the weights quantised for
 * the backward, and with recompute the activations are recomputed from x and the weights, so in
 * either case x and the weights must be unchanged since that moe_fwd).
 * Outputs (all overwritten, never accumulated):
 *   dx                 [T,H]
 *   dlogits            [T,E_total] fp32, zero outside each token's chosen experts
 *   dw_gate, dw_up     [E_local,F,H]
 *   dw_down            [E_local,H,F]
 * An expert that received no tokens gets exactly zero weight gradients. */
moe_status moe_bwd(const moe_desc* d, const void* dy, const void* x,
                   const void* w_gate, const void* w_up, const void* w_down, const void* saved,
                   void* dx, float* dlogits, void* dw_gate, void* dw_up, void* dw_down,
                   void* ws, size_t ws_bytes, void* stream);

/* Router projection in front of the layer: the linear router whose fp32 logits moe_fwd and
 * moe_route consume, and its backward. The pages fold the routing into the fused operation
 * ("Prime Mega MoE: kernel fuso per l'addestramento MoE" on "Prime Mega MoE: il kernel che
 * accelera il training AI del 55%") without saying how the logits arise; the library reads it as
 * the usual linear router without bias:
 *    logits[t, e]     = sum_h x[t, h] * w_router[e, h]        moe_router_fwd
 *    dw_router[e, h]  = sum_t dlogits[t, e] * x[t, h]         moe_router_bwd (overwritten)
 *    dx[t, h]        += sum_e dlogits[t, e] * w_router[e, h]  moe_router_bwd (accumulated)
 * w_router and dw_router are [E_total, H] (out x in, like the experts' weights); x and dx as in
 * the layer; logits and dlogits [T, E_total] fp32. Passing moe_bwd's dx and dlogits to
 * moe_router_bwd gives the gradient of the whole x -> router -> layer composition. In an expert
 * share, dlogits is the share's contribution and the call is linear in it, so the shares' calls
 * add up to the full gradient.
 * Arithmetic: bf16 MFMA with fp32 accumulation. Up to 256 experts the forward is one workgroup per
 * 64 tokens over all of H (the kernel moe_fwd_router uses, so the logits are bitwise the same);
 * beyond that, and for the contraction over the tokens (dw_router), the sums are split into slices
 * whose fp32 partial sums are added in a fixed order. The backward multiplies a bf16 copy of
 * dlogits, and dx is read, added to in fp32 and rounded once.
 * In MOE_MODE_FP32 (the test mode) x, w_router, dx and dw_router are fp32 and every output is a
 * plain fp32 sum in a fixed order. No atomics: results are bitwise reproducible.
 * Modes: all four (MXFP8 and FP8_BWD take bf16 I/O; the projection itself stays bf16). Every
 * tensor pointer needs 16-byte alignment except dlogits (4 bytes); ws needs 256. The workspace
 * sizes come from moe_query_router_sizes (host-only); its contents need not be preserved. */
moe_status moe_query_router_sizes(const moe_desc* d, size_t* fwd_ws, size_t* bwd_ws);
moe_status moe_router_fwd(const moe_desc* d, const void* x, const void* w_router, float* logits,
                          void* ws, size_t ws_bytes, void* stream);
moe_status moe_router_bwd(const moe_desc* d, const void* x, const void* w_router,
                          const float* dlogits, void* dx, void* dw_router, void* ws,
                          size_t ws_bytes, void* stream);

/* Byte offsets of the routing results inside `saved`.
 *   idx       int32 [T*k]      chosen experts, slot order (logit desc, index asc)
 *   weight    float [T*k]      renormalised routing weights
 *   counts    int32 [E_local]  pairs per local expert
 *   offsets   int32 [E_local+1] exclusive prefix sum of counts (offsets[E_local] = P)
 *   perm      int32 [T*k]      first P entries: pair ids t*k+j sorted by (expert, pair id)
 *   pair_pos  int32 [T*k]      position of pair t*k+j in perm, -1 if its expert is not local
 * and, in the MX modes without recompute (0 in the others), the MXFP8 operands the forward leaves
 * for the backward, each an e4m3 byte array with its e8m0 scale bytes:
 *   qoff      int32 [E_local+1] first column of each expert's segment in the pair-contiguous
 *                              copies; each segment is padded with zeros to a multiple of 128
 *   qcols     (value)          column count Q of the pair-contiguous copies
 *   hwt, hwt_scales            w*h transposed, [F, Q], blocks of 32 along each expert's pairs;
 *                              scales K-tile-major, [Q/128, F, 4]: the byte of row f, pair
 *                              column q at ((q/128) F + f) 4 + (q/32) % 4
 *   wdt, wdt_scales            (MXFP8) W_down[e] along H, transposed: [E_local, F, H], [E_local, F, H/32]
 *   wgut, wgut_scales          (MXFP8) [W_gate[e]^T | W_up[e]^T] along F: [E_local, H, 2F],
 *                              [E_local, H, 2F/32]
 * Host-only pointer arithmetic, for tests and tools. */
typedef struct {
  size_t idx, weight, counts, offsets, perm, pair_pos;
  size_t qoff, qcols, hwt, hwt_scales, wdt, wdt_scales, wgut, wgut_scales;
} moe_saved_offsets;
moe_status moe_saved_layout(const moe_desc* d, moe_saved_offsets* out);

/* MXFP8 quantisation of one bf16 matrix in [rows, cols] (row-major), with the element and scale
 * rules of MOE_MODE_MXFP8. It is the kernel the MX modes use on x, dy and the weights, exposed so
 * that it can be checked alone.
 *   axis = 1: blocks of 32 along each row. q [rows, cols] e4m3 bytes, scales [rows, cols/32]
 *             e8m0 bytes. cols % 32 == 0.
 *   axis = 0: blocks of 32 down each column, written transposed. q [cols, rows],
 *             scales [cols, rows/32]. rows % 128 == 0, cols % 64 == 0.
 * in and q need 16-byte alignment, scales 4-byte alignment; rows*cols < 2^34. Errors as
 * elsewhere (nothing is enqueued on error). */
moe_status moe_mx_quantize(const void* in, int64_t rows, int64_t cols, int axis, uint8_t* q,
                           uint8_t* scales, void* stream);

/* Blockwise FP8 quantisation of one bf16 matrix in [rows, cols] (row-major) with the rules of
 * MOE_MODE_FP8: the kernels that mode uses on x, dy and the weights, exposed so that they can be
 * checked alone. Scales keep the MXFP8 layout, one e8m0 byte per 32 elements along the blocked
 * axis, each block's scale repeated over its 32-element groups.
 *   weight = 0: an activation operand, blocks of 128 along each row. q [rows, cols] e4m3 bytes,
 *               scales [rows, cols/32]; qt and scales_t are unused (may be null). cols % 128 == 0.
 *   weight = 1: a weight matrix, one scale per 128 x 128 tile. q [rows, cols] and
 *               scales [rows, cols/32] hold the row orientation; qt [cols, rows] and
 *               scales_t [cols, rows/32] the transposed one, with the same scales.
 *               rows % 128 == 0, cols % 128 == 0.
 * in, q and qt need 16-byte alignment, the scale arrays 4-byte alignment; rows*cols < 2^34.
 * Errors as elsewhere (nothing is enqueued on error). */
moe_status moe_fp8_block_quantize(const void* in, int64_t rows, int64_t cols, int weight, uint8_t* q,
                                  uint8_t* scales, uint8_t* qt, uint8_t* scales_t, void* stream);

/* Static description of a status code. */
const char* moe_status_string(moe_status s);
/* Detail of the last error on the calling thread (empty string if none). */
const char* moe_last_error(void);

/* Kernel timing with HIP events, for measurement tools. While enabled, every kernel the
 * library launches is bracketed by two events recorded on the launch stream. The library
 * creates them up front, `max_launches` pairs, and reuses them. Launches beyond that are not
 * recorded. moe_profile_enable() clears earlier records. While enabled, the backward also
 * keeps its weight-gradient GEMMs on the launch stream (otherwise they run on a second stream of
 * the device, overlapping the dH and dgrad GEMMs), so that each duration is that kernel's alone.
 * moe_profile_collect() waits for the recorded events and sums each kernel's durations.
 * Kernel names are returned by index: moe_profile_kernel(i, &name, &launches, &total_ms)
 * gives MOE_ERR_INVALID_ARG once i runs past the last kernel. */
moe_status moe_profile_enable(int max_launches);
moe_status moe_profile_disable(void);
moe_status moe_profile_collect(void);
moe_status moe_profile_kernel(int i, const char** name, int* launches, double* total_ms);

/* Version string of the library build. */
const char* moe_version(void);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H */
