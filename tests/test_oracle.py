"""Pins of the float64 oracle against things other than itself (CPU only).

Each test checks the oracle against one of the following:
 * a brute-force loop;
 * a closed form;
 * torch's functional ops and autograd (float64, CPU);
 * central finite differences;
 * an invariant of the mathematics.
The planted-mistake tests at the end show that the pins catch the plausible slips:
 * a dropped term in dSwiGLU;
 * a wrong sign in the router gradient;
 * a transposed down-projection weight;
 * a wrong tie-break.
"""
import math

import numpy as np
import pytest
import scipy.special
import torch
import torch.nn.functional as Fn

import oracle
import oracle.moe_oracle as om
from mixture_experts_layer_32_amd import inputs


def small_layer(T=24, H=12, F=6, E=5, k=2, seed=7, zipf=0.0):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, H))
    logits = rng.standard_normal((T, E)) - zipf * np.log(np.arange(1, E + 1))[None, :]
    wg = rng.standard_normal((E, F, H)) / math.sqrt(H)
    wu = rng.standard_normal((E, F, H)) / math.sqrt(H)
    wd = rng.standard_normal((E, H, F)) / math.sqrt(F)
    dy = rng.standard_normal((T, H))
    return dict(x=x, logits=logits, wg=wg, wu=wu, wd=wd, dy=dy, k=k)


# ------------------------------------------------------------------------------------ routing

def brute_topk(row, k):
    """k passes of 'largest remaining value, lowest index on ties', in plain Python."""
    chosen = []
    for _ in range(k):
        best = None
        for e, v in enumerate(row):
            if e in chosen:
                continue
            if best is None or v > row[best]:
                best = e
        chosen.append(best)
    return chosen


@pytest.mark.parametrize("k", [1, 2, 3, 8])
def test_topk_matches_bruteforce_with_planted_ties(k):
    rng = np.random.default_rng(3)
    T, E = 40, 12
    lg = rng.integers(-3, 4, size=(T, E)).astype(np.float32)   # many exact ties
    lg[0] = 0.0
    lg[1, ::2] = -0.0                                            # -0.0 ties +0.0
    lg[2] = np.float32(1.5)
    idx = oracle.topk_select(lg, k)
    for t in range(T):
        assert list(idx[t]) == brute_topk([float(v) for v in lg[t]], k), t


def test_route_invariants_and_stable_order():
    L = small_layer(T=50, E=7, k=3)
    r = oracle.route(L["logits"], 3)
    T, k = 50, 3
    assert r["counts"].sum() == T * k
    assert sorted(r["perm"].tolist()) == list(range(T * k))            # bijection
    assert np.array_equal(r["pair_pos"][r["perm"]], np.arange(T * k))  # inverse
    # order: by (expert, pair id), checked against Python's tuple sort
    want = sorted(range(T * k), key=lambda p: (int(r["idx"].reshape(-1)[p]), p))
    assert r["perm"].tolist() == want
    for e in range(7):
        seg = r["perm"][r["offsets"][e]:r["offsets"][e + 1]]
        assert np.all(r["idx"].reshape(-1)[seg] == e)


def test_route_expert_share_keeps_only_local_pairs():
    L = small_layer(T=60, E=8, k=2)
    full = oracle.route(L["logits"], 2)
    sh = oracle.route(L["logits"], 2, e0=3, e_local=2)
    flat = full["idx"].reshape(-1)
    local = np.nonzero((flat >= 3) & (flat < 5))[0]
    assert sh["counts"].sum() == local.size
    assert sorted(sh["perm"].tolist()) == local.tolist()
    assert np.all(sh["pair_pos"][np.setdiff1d(np.arange(120), local)] == -1)
    assert np.array_equal(sh["w"], full["w"])        # weights stay renormalised over all k


def test_permute_then_unpermute_is_identity():
    L = small_layer(T=33, E=6, k=4)
    r = oracle.route(L["logits"], 4)
    x = L["x"]
    xp = x[r["perm"] // 4]                      # dispatch: expert-contiguous rows
    back = np.zeros((33 * 4, x.shape[1]))
    back[r["perm"]] = xp                        # undo the permutation
    assert np.array_equal(back.reshape(33, 4, -1), np.repeat(x[:, None, :], 4, axis=1))


def test_weights_against_scipy_softmax_then_renormalise():
    L = small_layer(T=30, E=9, k=4)
    idx = oracle.topk_select(L["logits"], 4)
    w = oracle.renormalised_weights(L["logits"], idx)
    p = scipy.special.softmax(L["logits"], axis=1)
    ps = np.take_along_axis(p, idx, axis=1)
    np.testing.assert_allclose(w, ps / ps.sum(1, keepdims=True), rtol=1e-13, atol=0)
    np.testing.assert_allclose(w.sum(1), 1.0, rtol=0, atol=1e-15)


def test_weights_special_cases():
    lg = np.random.default_rng(0).standard_normal((10, 6))
    assert np.all(oracle.renormalised_weights(lg, oracle.topk_select(lg, 1)) == 1.0)
    z = np.zeros((4, 8))
    assert np.all(oracle.renormalised_weights(z, oracle.topk_select(z, 4)) == 0.25)


# ------------------------------------------------------------------------------------ forward

def brute_forward(x, logits, wg, wu, wd, k):
    """Pure-Python loops with math.exp: routing, SwiGLU experts, weighted combine."""
    T, H = len(x), len(x[0])
    F = len(wg[0])
    y = [[0.0] * H for _ in range(T)]
    for t in range(T):
        sel = brute_topk(list(logits[t]), k)
        m = max(logits[t][e] for e in sel)
        z = [math.exp(logits[t][e] - m) for e in sel]
        for j, e in enumerate(sel):
            w = z[j] / sum(z)
            h = []
            for f in range(F):
                a = sum(wg[e][f][c] * x[t][c] for c in range(H))
                b = sum(wu[e][f][c] * x[t][c] for c in range(H))
                h.append(a / (1.0 + math.exp(-a)) * b)
            for c in range(H):
                y[t][c] += w * sum(wd[e][c][f] * h[f] for f in range(F))
    return np.array(y)


def test_forward_matches_bruteforce_loops():
    L = small_layer(T=7, H=5, F=3, E=4, k=2)
    y, _ = oracle.forward(L["x"], L["logits"], L["wg"], L["wu"], L["wd"], 2)
    yb = brute_forward(L["x"].tolist(), L["logits"].tolist(), L["wg"].tolist(),
                       L["wu"].tolist(), L["wd"].tolist(), 2)
    np.testing.assert_allclose(y, yb, rtol=1e-12, atol=1e-14)


def test_forward_closed_form_hand_example():
    """Two experts, T=1, H=2, F=1, k=2, worked by hand.

    With logits (0.5, 0), w = (sigmoid(0.5), 1 - sigmoid(0.5)).
    Expert 0: a=1, b=2, so h = 2 silu(1) and o0 = (h, -h).
    Expert 1: a=2, b=1, so h = silu(2) and o1 = (h, h).
    """
    x = np.array([[1.0, 2.0]])
    lg = np.array([[0.5, 0.0]])
    wg = np.array([[[1.0, 0.0]], [[0.0, 1.0]]])
    wu = np.array([[[0.0, 1.0]], [[1.0, 0.0]]])
    wd = np.array([[[1.0], [-1.0]], [[1.0], [1.0]]])
    y, _ = oracle.forward(x, lg, wg, wu, wd, 2)
    s = lambda z: 1.0 / (1.0 + math.exp(-z))
    w0 = s(0.5)
    h0, h1 = 2.0 * s(1.0), 2.0 * s(2.0)
    np.testing.assert_allclose(y[0], [w0 * h0 + (1 - w0) * h1, -w0 * h0 + (1 - w0) * h1],
                               rtol=1e-15)
    # backward with dY = (1, 0):
    #   u0 = 1  -> g0 = h0, dh0 = w0, da0 = w0*2*silu'(1), db0 = w0*silu(1), dWd0 = w0*dY*h0
    #   u1 = 1  -> g1 = h1, dh1 = w1, da1 = w1*1*silu'(2), db1 = w1*silu(2)
    g, _ = oracle.backward(np.array([[1.0, 0.0]]), x, lg, wg, wu, wd, 2)
    ds = lambda z: s(z) * (1 + z * (1 - s(z)))
    w1 = 1 - w0
    da0, db0 = w0 * 2 * ds(1.0), w0 * s(1.0)
    da1, db1 = w1 * ds(2.0), w1 * 2 * s(2.0)
    np.testing.assert_allclose(g["dx"][0], [da0 + db1, db0 + da1], rtol=1e-14)
    gbar = w0 * h0 + w1 * h1
    np.testing.assert_allclose(g["dlogits"][0], [w0 * (h0 - gbar), w1 * (h1 - gbar)], rtol=1e-13)
    np.testing.assert_allclose(g["dwd"][0], [[w0 * h0], [0.0]], rtol=1e-15)
    np.testing.assert_allclose(g["dwg"][1], [[da1 * 1.0, da1 * 2.0]], rtol=1e-14)
    np.testing.assert_allclose(g["dwu"][0], [[db0 * 1.0, db0 * 2.0]], rtol=1e-14)


def torch_swiglu(x, wg, wu, wd):
    return Fn.linear(Fn.silu(Fn.linear(x, wg)) * Fn.linear(x, wu), wd)


def test_single_expert_is_plain_swiglu_ffn():
    L = small_layer(T=20, H=16, F=8, E=1, k=1)
    y, _ = oracle.forward(L["x"], L["logits"], L["wg"], L["wu"], L["wd"], 1)
    t = lambda a: torch.from_numpy(np.asarray(a, np.float64))
    yt = torch_swiglu(t(L["x"]), t(L["wg"][0]), t(L["wu"][0]), t(L["wd"][0])).numpy()
    np.testing.assert_allclose(y, yt, rtol=1e-12, atol=1e-13)


def test_all_experts_equal_weights_is_dense_ffn():
    """k = E with equal logits: y = (1/E) * one wide SwiGLU FFN over the concatenated experts."""
    L = small_layer(T=15, H=10, F=4, E=6, k=6)
    lg = np.zeros((15, 6))
    y, _ = oracle.forward(L["x"], lg, L["wg"], L["wu"], L["wd"], 6)
    t = lambda a: torch.from_numpy(np.asarray(a, np.float64))
    wg = t(L["wg"]).reshape(6 * 4, 10)
    wu = t(L["wu"]).reshape(6 * 4, 10)
    wd = t(L["wd"]).permute(1, 0, 2).reshape(10, 6 * 4) / 6.0
    np.testing.assert_allclose(y, torch_swiglu(t(L["x"]), wg, wu, wd).numpy(), rtol=1e-12, atol=1e-13)


def test_forward_invariants():
    L = small_layer(T=18, E=5, k=2)
    f = lambda **kw: oracle.forward(**{**dict(x=L["x"], logits=L["logits"], wg=L["wg"], wu=L["wu"],
                                              wd=L["wd"], k=2), **kw})[0]
    y = f()
    assert np.all(f(x=np.zeros_like(L["x"])) == 0.0)
    np.testing.assert_allclose(f(wd=2.0 * L["wd"]), 2.0 * y, rtol=1e-14)
    p = np.random.default_rng(1).permutation(18)
    np.testing.assert_allclose(f(x=L["x"][p], logits=L["logits"][p]), y[p], rtol=1e-13, atol=1e-15)


# ------------------------------------------------------------------------------------ backward

def torch_layer_grads(L):
    """Dense-masked MoE in torch float64. Selection comes from torch.topk and is held constant.

    The routing weights are torch.softmax over the selected logits. Gradients come from
    autograd.
    """
    t = lambda a: torch.tensor(np.asarray(a, np.float64), requires_grad=True)
    x, lg, wg, wu, wd = t(L["x"]), t(L["logits"]), t(L["wg"]), t(L["wu"]), t(L["wd"])
    k = L["k"]
    idx = torch.topk(lg.detach(), k, dim=1).indices
    w = torch.softmax(torch.gather(lg, 1, idx), dim=1)
    y = torch.zeros_like(x)
    for e in range(wg.shape[0]):
        me = (w * (idx == e)).sum(1, keepdim=True)
        y = y + me * torch_swiglu(x, wg[e], wu[e], wd[e])
    (y * torch.from_numpy(np.asarray(L["dy"], np.float64))).sum().backward()
    return dict(y=y.detach().numpy(), dx=x.grad.numpy(), dlogits=lg.grad.numpy(),
                dwg=wg.grad.numpy(), dwu=wu.grad.numpy(), dwd=wd.grad.numpy())


def oracle_all(L, **kw):
    args = dict(x=L["x"], logits=L["logits"], wg=L["wg"], wu=L["wu"], wd=L["wd"], k=L["k"])
    args.update(kw)
    y, _ = oracle.forward(**args)
    g, r = oracle.backward(dy=L["dy"], **args)
    return dict(y=y, **{n: g[n] for n in ("dx", "dlogits", "dwg", "dwu", "dwd")})


@pytest.mark.parametrize("shape", [dict(T=24, H=12, F=6, E=5, k=2), dict(T=9, H=8, F=4, E=8, k=8),
                                   dict(T=31, H=6, F=10, E=3, k=1)])
def test_against_torch_autograd(shape):
    L = small_layer(**shape)
    o, tt = oracle_all(L), torch_layer_grads(L)
    for name in o:
        np.testing.assert_allclose(o[name], tt[name], rtol=1e-11, atol=1e-12, err_msg=name)


def fd_errors(L, eps=1e-5, seed=0):
    """Max relative error of <grad, v> against central differences of <dY, y> per input."""
    rng = np.random.default_rng(seed)
    base = dict(x=L["x"], logits=L["logits"], wg=L["wg"], wu=L["wu"], wd=L["wd"])
    g, _ = oracle.backward(L["dy"], k=L["k"], **base)
    gmap = dict(x="dx", logits="dlogits", wg="dwg", wu="dwu", wd="dwd")
    errs = {}
    for name, gname in gmap.items():
        v = rng.standard_normal(np.shape(base[name]))
        lp = oracle.forward(k=L["k"], **{**base, name: base[name] + eps * v})[0]
        lm = oracle.forward(k=L["k"], **{**base, name: base[name] - eps * v})[0]
        fd = np.sum(L["dy"] * (lp - lm)) / (2 * eps)
        an = np.sum(g[gname] * v)
        errs[name] = abs(fd - an) / max(abs(an), 1e-30)
    return errs


def routing_gap_ok(logits, k, margin):
    s = -np.sort(-np.asarray(logits, np.float64), axis=1)
    return np.all(s[:, k - 1] - s[:, k] > margin) if k < s.shape[1] else True


@pytest.mark.parametrize("shape", [dict(T=16, H=8, F=5, E=6, k=2), dict(T=10, H=6, F=4, E=4, k=3)])
def test_finite_differences(shape):
    L = small_layer(**shape)
    assert routing_gap_ok(L["logits"], L["k"], 1e-3)    # perturbation cannot change selection
    errs = fd_errors(L)
    assert max(errs.values()) < 1e-7, errs


def test_backward_invariants():
    L = small_layer(T=40, E=6, k=3)
    g = oracle_all(L)
    np.testing.assert_allclose(g["dlogits"].sum(1), 0.0, atol=1e-14)
    r = oracle.route(L["logits"], 3)
    mask = np.ones_like(g["dlogits"], bool)
    np.put_along_axis(mask, r["idx"], False, axis=1)
    assert np.all(g["dlogits"][mask] == 0.0)
    L1 = small_layer(T=12, E=1, k=1)
    assert np.all(oracle_all(L1)["dlogits"] == 0.0)
    # an expert nobody picks has exactly zero weight gradients
    L2 = small_layer(T=20, E=5, k=2)
    L2["logits"][:, 4] = -50.0
    g2 = oracle_all(L2)
    for n in ("dwg", "dwu", "dwd"):
        assert np.all(g2[n][4] == 0.0)


def test_expert_shares_add_up_to_the_full_layer():
    L = small_layer(T=45, E=8, k=3)
    full = oracle_all(L)
    acc = {n: 0.0 for n in ("y", "dx", "dlogits")}
    for e0 in range(0, 8, 2):
        sl = slice(e0, e0 + 2)
        part = oracle_all(L, wg=L["wg"][sl], wu=L["wu"][sl], wd=L["wd"][sl], e0=e0, e_local=2)
        for n in acc:
            acc[n] = acc[n] + part[n]
        for n in ("dwg", "dwu", "dwd"):
            np.testing.assert_allclose(part[n], full[n][sl], rtol=1e-13, atol=1e-15)
    for n in acc:
        np.testing.assert_allclose(acc[n], full[n], rtol=1e-12, atol=1e-13, err_msg=n)


def test_sampled_rows_and_experts_match_full():
    L = small_layer(T=40, E=6, k=2)
    full = oracle_all(L)
    toks = [0, 7, 39]
    s = oracle.token_rows(toks, L["dy"], L["x"], L["logits"], L["wg"], L["wu"], L["wd"], 2)
    for n in ("y", "dx", "dlogits"):
        np.testing.assert_allclose(s[n], full[n][toks], rtol=1e-12, atol=1e-14)
    for e in (0, 5):
        dg, du, dd = oracle.expert_grads(e, L["dy"], L["x"], L["logits"], L["wg"][e], L["wu"][e],
                                         L["wd"][e], 2)
        np.testing.assert_allclose(dg, full["dwg"][e], rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(du, full["dwu"][e], rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(dd, full["dwd"][e], rtol=1e-12, atol=1e-14)


def test_tiny_workload_against_torch_autograd():
    """The tiny workload at its real size (T=256, H=256, E=8, F=128, k=2)."""
    cfg = inputs.CONFIGS["tiny"]
    L = inputs.make_layer(cfg)
    L["k"] = cfg.k
    o, tt = oracle_all(L), torch_layer_grads(L)
    for name in o:
        assert oracle.rel_frobenius(o[name], tt[name]) < 1e-12, name


# ------------------------------------------------------------------------------------ the pins bite

def test_planted_mistake_dsilu_dropped_term_is_caught(monkeypatch):
    monkeypatch.setattr(om, "dsilu", lambda z: om.sigmoid(z))          # forgets z*s*(1-s)
    errs = fd_errors(small_layer(T=16, H=8, F=5, E=6, k=2))
    assert errs["x"] > 1e-3 and errs["wg"] > 1e-3


def test_planted_mistake_router_sign_is_caught(monkeypatch):
    real = om.router_grad
    monkeypatch.setattr(om, "router_grad", lambda r, g, E: -real(r, g, E))
    errs = fd_errors(small_layer(T=16, H=8, F=5, E=6, k=2))
    assert errs["logits"] > 1.0


def test_planted_mistake_transposed_down_weight_is_caught(monkeypatch):
    real = om.expert_forward

    def bad(xr, wg_e, wu_e, wd_e):                     # uses Wd instead of Wd^T (H == F here)
        a, b, h, _ = real(xr, wg_e, wu_e, wd_e)
        return a, b, h, h @ np.asarray(wd_e, np.float64)
    monkeypatch.setattr(om, "expert_forward", bad)
    L = small_layer(T=10, H=6, F=6, E=3, k=2)
    y, _ = oracle.forward(L["x"], L["logits"], L["wg"], L["wu"], L["wd"], 2)
    yb = brute_forward(L["x"].tolist(), L["logits"].tolist(), L["wg"].tolist(),
                       L["wu"].tolist(), L["wd"].tolist(), 2)
    assert np.max(np.abs(y - yb)) > 1e-3


def test_planted_mistake_tie_break_is_caught(monkeypatch):
    def high_index_first(lg, k):                        # ties go to the higher index
        lg = np.asarray(lg, np.float64)
        E = lg.shape[1]
        return (E - 1 - np.argsort(-lg[:, ::-1], axis=1, kind="stable"))[:, :k]
    monkeypatch.setattr(om, "topk_select", high_index_first)
    lg = np.array([[0.0, 1.0, 1.0, 0.0, 1.0]])
    assert list(om.route(lg, 2)["idx"][0]) != brute_topk(lg[0].tolist(), 2)


# ---------------------------------------------------------------------------- the parity metric
# rel_frobenius decides every parity verdict, so it is pinned against values worked out by hand.

def test_rel_frobenius_hand_values():
    # ref = [3, 4] (norm 5), got = [3, 5]: the difference [0, 1] has norm 1, so the error is 1/5.
    # Dividing by ||got|| = sqrt(34) would give 0.1715, the squared ratio 0.04.
    assert oracle.rel_frobenius(np.array([3.0, 5.0]), np.array([3.0, 4.0])) == pytest.approx(0.2, abs=1e-15)
    # the arguments are not symmetric: got = [3, 4], ref = [3, 5] gives 1/sqrt(34)
    assert oracle.rel_frobenius(np.array([3.0, 4.0]), np.array([3.0, 5.0])) == pytest.approx(1 / math.sqrt(34),
                                                                                              abs=1e-15)
    # a matrix takes the Frobenius norm, not the spectral one: ref = diag(3, 4) has Frobenius norm 5
    # (spectral 4); a difference of 1 in one element gives 0.2 (0.25 with spectral norms)
    ref = np.diag([3.0, 4.0])
    got = ref + np.array([[1.0, 0.0], [0.0, 0.0]])
    assert oracle.rel_frobenius(got, ref) == pytest.approx(0.2, abs=1e-15)
    # every element counts: ref all ones in 2x3 (norm sqrt 6), got off by 1 in two places -> sqrt(2/6)
    ref = np.ones((2, 3))
    got = ref.copy()
    got[0, 2] = 2.0
    got[1, 0] = 0.0
    assert oracle.rel_frobenius(got, ref) == pytest.approx(math.sqrt(2.0 / 6.0), abs=1e-15)
    # scale-free: the same relative difference at 2^40 and 2^-40
    for s in (2.0 ** 40, 2.0 ** -40):
        assert oracle.rel_frobenius(s * np.array([3.0, 5.0]), s * np.array([3.0, 4.0])) == pytest.approx(0.2)


def test_rel_frobenius_zero_reference():
    z = np.zeros((3, 4))
    assert oracle.rel_frobenius(z, z) == 0.0
    # -0.0 counts as zero
    assert oracle.rel_frobenius(-z, z) == 0.0
    got = z.copy()
    got[1, 2] = 1e-30
    assert oracle.rel_frobenius(got, z) == float("inf")


def test_rel_frobenius_reads_float32_and_bf16_bits_exactly():
    # float32 inputs are widened to float64 before any arithmetic: 1 + 2^-23 vs 1 differs by 2^-23
    got = np.array([1.0 + 2.0 ** -23], dtype=np.float32)
    ref = np.array([1.0], dtype=np.float32)
    assert oracle.rel_frobenius(got, ref) == 2.0 ** -23
    # a torch bf16 tensor converted through float32 keeps its value
    t = torch.tensor([1.0078125, 2.0], dtype=torch.bfloat16)       # 1 + 2^-7 is exact in bf16
    assert oracle.rel_frobenius(t.float().numpy(), np.array([1.0, 2.0])) == pytest.approx(
        2.0 ** -7 / math.sqrt(5.0), rel=1e-15)
