"""Float64 CPU oracle of the fused MoE layer, forward and backward. TEST INFRASTRUCTURE ONLY.

Only the test suite, the package's smoke check and the benchmark's CPU-baseline leg may import
this module. The HIP library never calls it. It shares no code with the HIP path, and it imports
nothing from the product package.

What the layer computes comes from three news pages about Prime Intellect's "Prime Mega MoE"
(an extension of DeepSeek's "Mega MoE" kernel).
 * Dispatch of tokens to experts, the experts' linear layers, SwiGLU and the combine of the
   results happen in one fused call: "A Magia da Fusão" on "IA: MoE Kernel 3x Mais Rápido
   Chegou!", and "Qué se ha publicado" on the ai-daily-news.org page.
 * Experts are gated SwiGLU without biases: "Detalhes Técnicos Rápidos" on the first page.
 * 128 experts with top-8 routing: "Os Números que Impressionam" on the first page, and
   "Analisi dei kernel layer" on "Prime Mega MoE: il kernel che accelera il training AI
   del 55%".
 * The backward pass is the part Prime added: "Afinal, o que é esse Prime Mega MoE?" on the
   first page.
The pages give no formulas. Where they are silent, this module takes the plainest reading:
 * softmax routing over fp32 logits, top-k, renormalised over the chosen k;
 * ties go to the lower expert index;
 * silu(gate) * up;
 * a weighted sum in the combine;
 * no capacity limit and no token dropping.
Each function states its reading.

Arrays may arrive as float32, including bf16-exact values. Every computation converts them to
float64 before any arithmetic.

The router projection (router_forward, router_backward) produces the logits the layer consumes,
and takes its dlogits back.

Parity status: every function here is pinned by tests that do not go through this code:
 * brute-force loops;
 * closed forms;
 * torch's own functional ops and autograd;
 * central finite differences.
No function is "parity unpinned".

Quantised precision modes (mode="mxfp8": MXFP8 in both passes; mode="fp8_bwd": MXFP8 in the
backward only; mode="fp8": blockwise FP8 in both passes). Every GEMM operand is replaced by its
round trip (oracle/mx.py) along that GEMM's contraction axis:
    gate/up        x rows and W_gate, W_up along H
    down           (w * h) along F; W_down along F
    dH             dY rows along H; W_down along H
    down wgrad     dY and (w * h) along the expert's pairs, in the stable pair order, in blocks of 32
                   (fp8: 128) from the expert's first pair (the last block zero-padded)
    gate/up wgrad  da, db and x along the expert's pairs
    dgrad x        da, db along F; W_gate, W_up along F
MXFP8 blocks are 32 elements along the contraction axis. Blockwise FP8 uses blocks of 128 for the
activation operands and one scale per 128 x 128 tile of each expert weight matrix, whichever axis
the GEMM contracts, with a power-of-two scale that never saturates (oracle/mx.py).
Routing, softmax, SwiGLU, the router gradient and the combines stay exact.
Reading: the routing weight enters before the down projection (o' = W_down (w h)). Without
quantisation that is the same sum as weighting the expert output. In MX modes it fixes which
operand is quantised.
"""
from __future__ import annotations

import numpy as np

from . import mx


def _f64(a):
    return np.asarray(a, dtype=np.float64)


# ----------------------------------------------------------------------------------------------
# routing

def topk_select(logits, k):
    """Top-k expert indices per token, ordered by (logit descending, expert index ascending).

    Reading: the pages only say "top-8 routing". Selection is on the fp32 logits themselves.
    Softmax is monotone, so in exact arithmetic this is the same set as top-k over the
    probabilities. Ties go to the lower expert index, and -0.0 equals +0.0.
    """
    lg = _f64(logits)
    # a stable sort of the negated logits puts equal values in ascending index order
    order = np.argsort(-lg, axis=1, kind="stable")
    return order[:, :k].astype(np.int64)


def renormalised_weights(logits, idx):
    """w[t,j] = softmax over all experts, restricted to the chosen k and renormalised.

    The softmax normaliser cancels in the renormalisation, so
    w_tj = exp(l_{t,S_tj} - m_t) / sum_i exp(l_{t,S_ti} - m_t), with m_t the largest chosen
    logit. No epsilon is added to the denominator.
    """
    lg = _f64(logits)
    sel = np.take_along_axis(lg, idx, axis=1)
    z = np.exp(sel - sel.max(axis=1, keepdims=True))
    return z / z.sum(axis=1, keepdims=True)


def route(logits, k, e0=0, e_local=None):
    """Full routing metadata for the experts [e0, e0+e_local).

    Returns a dict:
      idx      [T,k]   chosen experts (global ids)
      w        [T,k]   renormalised weights
      counts   [El]    pairs routed to each local expert
      offsets  [El+1]  exclusive prefix sum of counts
      perm     [P]     pair ids (t*k + j) sorted by (local expert, pair id): a stable counting
                       sort, which is the "token sorting" the pages name as a cost
      pair_pos [T*k]   inverse of perm; -1 for pairs whose expert is not local
    """
    lg = _f64(logits)
    T, E = lg.shape
    el = E - e0 if e_local is None else e_local
    idx = topk_select(lg, k)
    w = renormalised_weights(lg, idx)
    flat = idx.reshape(-1)
    local = (flat >= e0) & (flat < e0 + el)
    pair_ids = np.nonzero(local)[0]
    experts = flat[pair_ids] - e0
    counts = np.bincount(experts, minlength=el).astype(np.int64)
    offsets = np.zeros(el + 1, np.int64)
    offsets[1:] = np.cumsum(counts)
    perm = pair_ids[np.argsort(experts, kind="stable")]
    pair_pos = np.full(T * k, -1, np.int64)
    pair_pos[perm] = np.arange(perm.size)
    return dict(idx=idx, w=w, counts=counts, offsets=offsets, perm=perm, pair_pos=pair_pos,
                k=k, e0=e0, el=el)


# ----------------------------------------------------------------------------------------------
# expert feed-forward (gated SwiGLU, no biases)

def sigmoid(z):
    return 1.0 / (1.0 + np.exp(-z))


def silu(z):
    return z * sigmoid(z)


def dsilu(z):
    """d/dz [z * sigmoid(z)] = sigmoid(z) * (1 + z * (1 - sigmoid(z)))."""
    s = sigmoid(z)
    return s * (1.0 + z * (1.0 - s))


def expert_forward(xr, wg_e, wu_e, wd_e):
    """One expert on its rows xr [n,H]: a = xr Wg^T, b = xr Wu^T, h = silu(a)*b, o = h Wd^T."""
    xr = _f64(xr)
    a = xr @ _f64(wg_e).T
    b = xr @ _f64(wu_e).T
    h = silu(a) * b
    o = h @ _f64(wd_e).T
    return a, b, h, o


def _fwd_quant(mode):
    """Operand quantiser kind of the forward GEMMs in `mode`: None (exact), "mx" or "blk"."""
    return {"mxfp8": "mx", "fp8": "blk"}.get(mode)


def _bwd_quant(mode):
    """Operand quantiser kind of the backward GEMMs in `mode`."""
    return {"mxfp8": "mx", "fp8_bwd": "mx", "fp8": "blk"}.get(mode)


def _qz(kind, v, axis, weight=False):
    """GEMM operand v quantised along `axis`, its contraction axis. kind None leaves it exact; "mx" is
    MXFP8 (blocks of 32); "blk" is blockwise FP8: blocks of 128 along the axis for an activation
    operand, 128 x 128 tiles for an expert's weight matrix (the same in both orientations)."""
    if not kind:
        return _f64(v)
    if kind == "blk":
        return mx.fp8_tile_quantize(v) if weight else mx.fp8_block_quantize(v, axis)
    return mx.mx_quantize(v, axis)


def expert_forward_q(xr, wr, wg_e, wu_e, wd_e, quant):
    """One expert with quantised operands (quant: "mx" or "blk"; True means "mx"). Returns a, b, h
    and o' = W_down (w h)."""
    quant = "mx" if quant is True else quant
    xq = _qz(quant, xr, 1)
    a = xq @ _qz(quant, wg_e, 1, weight=True).T
    b = xq @ _qz(quant, wu_e, 1, weight=True).T
    h = silu(a) * b
    o = _qz(quant, wr[:, None] * h, 1) @ _qz(quant, wd_e, 1, weight=True).T
    return a, b, h, o


def _expert_rows(r, i):
    """(pair ids, token ids, weights) of local expert i, in the stable pair order."""
    pairs = r["perm"][r["offsets"][i]:r["offsets"][i + 1]]
    return pairs, pairs // r["k"], r["w"].reshape(-1)[pairs]


# ----------------------------------------------------------------------------------------------
# forward

def forward(x, logits, wg, wu, wd, k, e0=0, e_local=None, mode=None):
    """y[t] = sum over the local chosen slots j of w_tj * FFN_{S_tj}(x_t).

    wg, wu [El,F,H] and wd [El,H,F] hold the local experts e0..e0+El-1. A token with no local
    slot gets y = 0. For a share of the experts, y is that share's partial sum; the layer output
    is the sum over shares.
    """
    x = _f64(x)
    T, H = x.shape
    r = route(logits, k, e0, e_local if e_local is not None else len(wg))
    y = np.zeros((T, H))
    for i in range(r["el"]):
        pairs, toks, wr = _expert_rows(r, i)
        if pairs.size == 0:
            continue
        if _fwd_quant(mode):
            _, _, _, o = expert_forward_q(x[toks], wr, wg[i], wu[i], wd[i], _fwd_quant(mode))
            y[toks] += o                    # the routing weight is inside o'
        else:
            _, _, _, o = expert_forward(x[toks], wg[i], wu[i], wd[i])
            y[toks] += wr[:, None] * o      # a token meets an expert at most once
    return y, r


# ----------------------------------------------------------------------------------------------
# backward

def backward(dy, x, logits, wg, wu, wd, k, e0=0, e_local=None, mode=None):
    """Gradients of L = <dY, y> with respect to x, the router logits and the expert weights.

    Per routed pair (t, j) with expert e and weight w = w_tj:
      u  = Wd[e]^T dY_t                   (dL/dh before the routing weight)
      g  = <u, h> = <dY_t, o_tj>         (dL/dw_tj)
      dh = w u
      da = dh * b * dsilu(a),  db = dh * silu(a)
      dWd[e] += (w dY_t) h^T,  dWg[e] += da x_t^T,  dWu[e] += db x_t^T
      dx_t   += Wg[e]^T da + Wu[e]^T db
    Router: dlogits[t, S_ti] = w_ti (g_ti - sum_j w_tj g_tj). Slots whose expert is not local
    have g = 0. Unchosen experts get 0. The index selection is piecewise constant and carries no
    gradient.
    Reading: the pages name only a backward pass (dgrad, wgrad, dSwiGLU and the router-weight
    gradient are the parts any such pass must produce). In the MX modes the backward GEMMs
    take MXFP8 operands as listed in the module docstring.
    """
    x, dy = _f64(x), _f64(dy)
    T, H = x.shape
    el = e_local if e_local is not None else len(wg)
    r = route(logits, k, e0, el)
    E = np.asarray(logits).shape[1]
    dx = np.zeros((T, H))
    g = np.zeros(T * k)
    dwg = np.zeros(np.shape(wg))
    dwu = np.zeros(np.shape(wu))
    dwd = np.zeros(np.shape(wd))
    for i in range(el):
        pairs, toks, wr = _expert_rows(r, i)
        if pairs.size == 0:
            continue
        gi, dwg[i], dwu[i], dwd[i], dxe = _expert_backward(x[toks], dy[toks], wr, wg[i], wu[i], wd[i], mode)
        g[pairs] = gi
        dx[toks] += dxe
    dlogits = router_grad(r, g.reshape(T, k), E)
    return dict(dx=dx, dlogits=dlogits, dwg=dwg, dwu=dwu, dwd=dwd, g=g.reshape(T, k)), r


def _expert_backward(xe, dye, wr, wg_i, wu_i, wd_i, mode):
    """(g, dWg, dWu, dWd, dx rows) of one expert's pairs, in the stable pair order."""
    qb = _bwd_quant(mode)
    if _fwd_quant(mode):
        a, b, h, _ = expert_forward_q(xe, wr, wg_i, wu_i, wd_i, _fwd_quant(mode))
    else:
        a, b, h, _ = expert_forward(xe, wg_i, wu_i, wd_i)
    u = _qz(qb, dye, 1) @ _qz(qb, wd_i, 0, weight=True)    # contraction over H
    g = np.sum(u * h, axis=1)
    dh = wr[:, None] * u
    da = dh * b * dsilu(a)
    db = dh * silu(a)
    hw = wr[:, None] * h
    if qb:                                                  # contraction over the pairs
        dwd = _qz(qb, dye, 0).T @ _qz(qb, hw, 0)
        xq = _qz(qb, xe, 0)
        dwg = _qz(qb, da, 0).T @ xq
        dwu = _qz(qb, db, 0).T @ xq
    else:
        dwd = (wr[:, None] * dye).T @ h
        dwg = da.T @ xe
        dwu = db.T @ xe
    dxe = (_qz(qb, da, 1) @ _qz(qb, wg_i, 0, weight=True)
           + _qz(qb, db, 1) @ _qz(qb, wu_i, 0, weight=True))                # contraction over F
    return g, dwg, dwu, dwd, dxe


# ----------------------------------------------------------------------------------------------
# router projection in front of the layer

def router_forward(x, wr):
    """Router logits l = x W_r^T, [T, E], with W_r [E, H] (out x in, like the experts' weights).

    The pages fold the routing into the fused call ("Prime Mega MoE: kernel fuso per
    l'addestramento MoE" on "Prime Mega MoE: il kernel che accelera il training AI del 55%") but
    do not say how the logits arise. Reading: the usual linear router, without bias. The routing
    above consumes fp32 logits; this returns them in float64, and the caller rounds them where it
    needs fp32 bits.
    """
    return _f64(x) @ _f64(wr).T


def router_backward(dlogits, x, wr):
    """Gradients of the router projection for dlogits [T, E]: dW_r = dlogits^T x [E, H], and the
    router's part of dx, dlogits W_r [T, H], which adds to the layer's own dx."""
    dl = _f64(dlogits)
    return dl.T @ _f64(x), dl @ _f64(wr)


def router_grad(r, g, E):
    """dlogits [T,E] from g[t,j] = dL/dw_tj through the renormalised softmax."""
    w = r["w"]
    T, k = w.shape
    dsel = w * (g - np.sum(w * g, axis=1, keepdims=True))
    dl = np.zeros((T, E))
    np.put_along_axis(dl, r["idx"], dsel, axis=1)
    return dl


# ----------------------------------------------------------------------------------------------
# sampled evaluation for full-size layers: each quantity below depends only on the pairs named

def token_rows(tokens, dy, x, logits, wg, wu, wd, k, e0=0, e_local=None, mode=None):
    """y, dx and dlogits rows of the given tokens. They need only those tokens' own pairs.

    In the MX modes, every quantised operand of these rows is blocked along a row (H or F), so
    the rows are still independent.
    """
    x, dy = _f64(x), _f64(dy)
    el = e_local if e_local is not None else len(wg)
    lg = _f64(logits)[np.asarray(tokens)]
    idx = topk_select(lg, k)
    w = renormalised_weights(lg, idx)
    n, H = len(tokens), x.shape[1]
    y = np.zeros((n, H))
    dx = np.zeros((n, H))
    g = np.zeros((n, k))
    qb, qf = _bwd_quant(mode), _fwd_quant(mode)
    for q, t in enumerate(tokens):
        for j in range(k):
            e = int(idx[q, j])
            if not (e0 <= e < e0 + el):
                continue
            i = e - e0
            wr = np.array([w[q, j]])
            if qf:
                a, b, h, o = expert_forward_q(x[t:t + 1], wr, wg[i], wu[i], wd[i], qf)
                y[q] += o[0]
            else:
                a, b, h, o = expert_forward(x[t:t + 1], wg[i], wu[i], wd[i])
                y[q] += w[q, j] * o[0]
            u = _qz(qb, dy[t:t + 1], 1) @ _qz(qb, wd[i], 0, weight=True)
            g[q, j] = np.sum(u * h)
            dh = w[q, j] * u
            da = dh * b * dsilu(a)
            db = dh * silu(a)
            dx[q] += (_qz(qb, da, 1) @ _qz(qb, wg[i], 0, weight=True)
                      + _qz(qb, db, 1) @ _qz(qb, wu[i], 0, weight=True))[0]
    rr = dict(w=w, idx=idx)
    return dict(y=y, dx=dx, dlogits=router_grad(rr, g, lg.shape[1]), idx=idx, w=w)


def expert_grads(i, dy, x, logits, wg_i, wu_i, wd_i, k, e0=0, e_local=None, r=None, mode=None):
    """dW_gate, dW_up, dW_down of local expert i. They need only that expert's rows."""
    x, dy = _f64(x), _f64(dy)
    if r is None:
        r = route(logits, k, e0, e_local)
    pairs, toks, wr = _expert_rows(r, i)
    F, H = np.shape(wg_i)
    if pairs.size == 0:
        return np.zeros((F, H)), np.zeros((F, H)), np.zeros((H, F))
    _, dwg, dwu, dwd, _ = _expert_backward(x[toks], dy[toks], wr, wg_i, wu_i, wd_i, mode)
    return dwg, dwu, dwd


def rel_frobenius(got, ref):
    """||got - ref||_F / ||ref||_F in float64. If ref is exactly zero, got must be zero too."""
    got, ref = _f64(got), _f64(ref)
    nr = np.linalg.norm(ref)
    if nr == 0.0:
        return 0.0 if not np.any(got) else float("inf")
    return float(np.linalg.norm(got - ref) / nr)
