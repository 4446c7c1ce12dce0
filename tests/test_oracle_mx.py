"""Pins of the oracle's MXFP8 emulation and MX precision modes (CPU only).

The quantiser is checked against things it does not share code with:
 * torch's float8_e4m3fn decode and cast;
 * brute-force nearest search over the 254 finite values;
 * closed forms of the block scale;
 * scale invariance.
The MX data flow of the layer is checked against a per-pair brute force whose quantiser is torch's
fp8 cast, and by the reductions each mode must satisfy.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import mx


def _torch_e4m3(v):
    """RNE cast to E4M3 by torch, for |v| <= 448."""
    return torch.from_numpy(np.asarray(v, np.float32)).to(torch.float8_e4m3fn).to(torch.float64).numpy()


def _torch_mx(v, axis):
    """MXFP8 round trip with torch's fp8 cast as the element quantiser (blocks of 32, zero-padded)."""
    x = np.moveaxis(np.asarray(v, np.float64), axis, -1)
    n = x.shape[-1]
    out = np.empty_like(x)
    for b0 in range(0, n, 32):
        blk = x[..., b0:b0 + 32]
        amax = np.abs(blk).max(axis=-1, keepdims=True)
        s = np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - 8
        s = np.where(amax > 0, np.clip(s, -127, 127), -127)
        sc = 2.0 ** s
        q = np.clip(blk / sc, -448, 448)
        # torch casts from float32: inputs are float32-exact, while float64 intermediates (h, da)
        # round to float32 first, which can move the fp8 choice only within 2^-24 of a midpoint
        # (no seeded case here lands there)
        out[..., b0:b0 + 32] = _torch_e4m3(q) * sc
    return np.moveaxis(out, -1, axis)


# ---------------------------------------------------------------------------------------------
# the element format

def test_e4m3_table_matches_torch_decode():
    codes = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    finite = np.sort(codes[np.isfinite(codes)])
    assert np.array_equal(np.sort(mx.e4m3_table()), finite)
    assert finite.max() == 448.0 and np.min(finite[finite > 0]) == 2.0 ** -9


def test_e4m3_round_matches_torch_cast_in_range():
    rng = np.random.default_rng(1)
    v = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.uniform(-3, 2.6, 20000),
                        rng.uniform(-448, 448, 5000)]).astype(np.float32)
    v = v[np.abs(v) <= 448]                 # torch's cast gives NaN beyond; this format saturates
    assert v.size > 20000
    assert np.array_equal(mx.e4m3_round(v), _torch_e4m3(v))


def test_e4m3_round_ties_to_even_and_nearest():
    tab = np.sort(np.unique(mx.e4m3_table()))
    pos = tab[tab >= 0]
    mids = (pos[:-1] + pos[1:]) / 2
    r = mx.e4m3_round(mids)
    # each midpoint goes to the neighbour whose code has an even mantissa (last bit zero)
    codes = {float(v): i for i, v in enumerate(pos)}   # positive codes are ordered like values
    for m, q, lo, hi in zip(mids, r, pos[:-1], pos[1:]):
        assert q in (lo, hi)
        assert codes[float(q)] % 2 == 0, (m, q)
    rng = np.random.default_rng(2)
    v = rng.uniform(-448, 448, 3000)
    near = tab[np.argmin(np.abs(v[:, None] - tab[None, :]), axis=1)]
    assert np.array_equal(mx.e4m3_round(v), near)


def test_e4m3_round_saturates():
    assert np.array_equal(mx.e4m3_round([449.0, 500.0, 1e30, -1e6]), [448.0, 448.0, 448.0, -448.0])
    assert mx.e4m3_round(0.0) == 0.0 and mx.e4m3_round(2.0 ** -11) == 0.0   # below half the min


# ---------------------------------------------------------------------------------------------
# the block scale

@pytest.mark.parametrize("p", [-20, -1, 0, 3, 15])
def test_block_scale_closed_form(p):
    amax = 2.0 ** p
    assert mx.block_scale_exponent(amax) == p - 8
    assert mx.block_scale_exponent(amax * 1.999) == p - 8
    assert mx.block_scale_exponent(amax * 2) == p - 7


def test_block_scale_zero_and_clamps():
    assert mx.block_scale_exponent(0.0) == -127
    assert mx.block_scale_exponent(2.0 ** 200) == 127
    assert mx.block_scale_exponent(2.0 ** -200) == -127
    z = mx.mx_quantize(np.zeros((3, 64)))
    assert np.array_equal(z, np.zeros((3, 64)))


def test_mx_quantize_exact_values_are_fixed_points():
    rng = np.random.default_rng(3)
    tab = mx.e4m3_table()
    el = rng.choice(tab[np.abs(tab) <= 256], size=(4, 96))
    el[:, ::32] = 256.0                                   # amax 256 puts the scale at 2^0
    sc = 2.0 ** rng.integers(-30, 30, size=(4, 3)).repeat(32, axis=1)
    v = el * sc
    assert np.array_equal(mx.mx_quantize(v, axis=1), v)


def test_mx_quantize_scale_invariance_and_error_bound():
    rng = np.random.default_rng(4)
    v = rng.standard_normal((8, 200))
    q = mx.mx_quantize(v, axis=1)
    for j in (-40, -3, 7, 60):
        assert np.array_equal(mx.mx_quantize(v * 2.0 ** j, axis=1), q * 2.0 ** j)
    # per element: half an ulp of a 3-bit mantissa, or saturation at 448 X
    deq, el, s = mx.mx_quantize(v, axis=1, return_parts=True)
    X = np.repeat(2.0 ** s, 32, axis=-1)[:, :200]
    sat = np.abs(v) / X > 448
    err = np.abs(deq - v)
    assert np.all(err[~sat] <= np.maximum(2.0 ** -4 * np.abs(v[~sat]), 2.0 ** -10 * X[~sat]) * (1 + 1e-12))
    assert np.array_equal(np.abs(deq[sat]), 448 * X[sat])


def test_mx_quantize_matches_torch_quantiser_and_axis():
    rng = np.random.default_rng(5)
    v = (rng.standard_normal((37, 70)) * 3).astype(np.float32)
    assert np.array_equal(mx.mx_quantize(v, axis=1), _torch_mx(v, 1))
    assert np.array_equal(mx.mx_quantize(v, axis=0), _torch_mx(v, 0))
    assert not np.array_equal(mx.mx_quantize(v, axis=0), mx.mx_quantize(v, axis=1))


def test_mx_quantize_pads_last_block_with_zeros():
    rng = np.random.default_rng(6)
    v = rng.standard_normal((3, 40))
    padded = np.concatenate([v, np.zeros((3, 24))], axis=1)
    assert np.array_equal(mx.mx_quantize(v, axis=1), mx.mx_quantize(padded, axis=1)[:, :40])


# ---------------------------------------------------------------------------------------------
# the layer in MX modes

def _tiny(seed=7, T=19, H=64, F=64, E=6, k=2):
    rng = np.random.default_rng(seed)
    f32 = lambda a: a.astype(np.float32).astype(np.float64)
    x = f32(rng.standard_normal((T, H)))
    dy = f32(rng.standard_normal((T, H)))
    lg = f32(rng.standard_normal((T, E)))
    wg = f32(rng.standard_normal((E, F, H)) / 8)
    wu = f32(rng.standard_normal((E, F, H)) / 8)
    wd = f32(rng.standard_normal((E, H, F)) / 8)
    return x, dy, lg, wg, wu, wd, k


def _brute_mx(x, dy, lg, wg, wu, wd, k, qfwd, qbwd):
    """Per token and slot loops; torch's fp8 cast is the quantiser. Wgrad operands are blocked along
    each expert's pairs in ascending pair order (token-major, then slot)."""
    T, H = x.shape
    E, F, _ = wg.shape
    Q = lambda on, v, ax: _torch_mx(v, ax) if on else v
    sg = lambda z: 1 / (1 + np.exp(-z))
    y = np.zeros((T, H))
    dx = np.zeros((T, H))
    g = np.zeros((T, k))
    rows = {e: [] for e in range(E)}
    for t in range(T):
        order = sorted(range(E), key=lambda e: (-lg[t, e], e))[:k]
        z = np.exp(lg[t, order] - lg[t, order].max())
        w = z / z.sum()
        for j, e in enumerate(order):
            xr = Q(qfwd, x[t:t + 1], 1)
            a = xr @ Q(qfwd, wg[e], 1).T
            b = xr @ Q(qfwd, wu[e], 1).T
            h = a * sg(a) * b
            y[t] += (Q(qfwd, w[j] * h, 1) @ Q(qfwd, wd[e], 1).T)[0]
            u = Q(qbwd, dy[t:t + 1], 1) @ Q(qbwd, wd[e], 0)
            g[t, j] = np.sum(u * h)
            dh = w[j] * u
            da = dh * b * sg(a) * (1 + a * (1 - sg(a)))
            db = dh * a * sg(a)
            dx[t] += (Q(qbwd, da, 1) @ Q(qbwd, wg[e], 0) + Q(qbwd, db, 1) @ Q(qbwd, wu[e], 0))[0]
            rows[e].append((t, w[j] * h[0], da[0], db[0]))
    dwg = np.zeros_like(wg)
    dwu = np.zeros_like(wu)
    dwd = np.zeros_like(wd)
    for e, rr in rows.items():
        if not rr:
            continue
        ts = [r[0] for r in rr]
        HW = np.array([r[1] for r in rr])
        DA = np.array([r[2] for r in rr])
        DB = np.array([r[3] for r in rr])
        dwd[e] = Q(qbwd, dy[ts], 0).T @ Q(qbwd, HW, 0)
        dwg[e] = Q(qbwd, DA, 0).T @ Q(qbwd, x[ts], 0)
        dwu[e] = Q(qbwd, DB, 0).T @ Q(qbwd, x[ts], 0)
    return y, dx, g, dwg, dwu, dwd


@pytest.mark.parametrize("mode", ["mxfp8", "fp8_bwd"])
def test_mx_modes_match_brute_force(mode):
    x, dy, lg, wg, wu, wd, k = _tiny(T=41)     # expert segments longer than one 32-pair block
    qf = mode == "mxfp8"
    y_b, dx_b, g_b, dwg_b, dwu_b, dwd_b = _brute_mx(x, dy, lg, wg, wu, wd, k, qf, True)
    y, _ = oracle.forward(x, lg, wg, wu, wd, k, mode=mode)
    gr, _ = oracle.backward(dy, x, lg, wg, wu, wd, k, mode=mode)
    # the brute force sums in another order; float64 round-off only, quantisation decisions agree
    for got, ref in ((y, y_b), (gr["dx"], dx_b), (gr["g"], g_b), (gr["dwg"], dwg_b), (gr["dwu"], dwu_b),
                     (gr["dwd"], dwd_b)):
        assert np.allclose(got, ref, rtol=1e-9, atol=1e-9)


def test_fp8_bwd_forward_is_the_exact_forward():
    x, dy, lg, wg, wu, wd, k = _tiny()
    y0, _ = oracle.forward(x, lg, wg, wu, wd, k)
    y1, _ = oracle.forward(x, lg, wg, wu, wd, k, mode="fp8_bwd")
    assert np.array_equal(y0, y1)


@pytest.mark.parametrize("mode", ["mxfp8", "fp8_bwd"])
def test_mx_modes_stay_close_to_exact(mode):
    """MXFP8 moves every output by a few per cent, not more, and not by nothing."""
    x, dy, lg, wg, wu, wd, k = _tiny(T=64)
    y0, _ = oracle.forward(x, lg, wg, wu, wd, k)
    g0, _ = oracle.backward(dy, x, lg, wg, wu, wd, k)
    y1, _ = oracle.forward(x, lg, wg, wu, wd, k, mode=mode)
    g1, _ = oracle.backward(dy, x, lg, wg, wu, wd, k, mode=mode)
    if mode == "mxfp8":
        assert 1e-3 < oracle.rel_frobenius(y1, y0) < 0.08
    for n in ("dx", "dlogits", "dwg", "dwu", "dwd"):
        assert 1e-3 < oracle.rel_frobenius(g1[n], g0[n]) < 0.1, n


@pytest.mark.parametrize("mode", ["mxfp8", "fp8_bwd"])
def test_mx_row_and_expert_helpers_agree_with_full_passes(mode):
    x, dy, lg, wg, wu, wd, k = _tiny(T=50, E=4, k=2)
    y, r = oracle.forward(x, lg, wg, wu, wd, k, mode=mode)
    gr, _ = oracle.backward(dy, x, lg, wg, wu, wd, k, mode=mode)
    toks = [0, 7, 33, 49]
    rows = oracle.token_rows(toks, dy, x, lg, wg, wu, wd, k, mode=mode)
    assert np.allclose(rows["y"], y[toks], rtol=1e-12, atol=1e-12)
    assert np.allclose(rows["dx"], gr["dx"][toks], rtol=1e-12, atol=1e-12)
    assert np.allclose(rows["dlogits"], gr["dlogits"][toks], rtol=1e-12, atol=1e-12)
    for i in range(4):
        dwg, dwu, dwd = oracle.expert_grads(i, dy, x, lg, wg[i], wu[i], wd[i], k, r=r, mode=mode)
        assert np.allclose(dwg, gr["dwg"][i], rtol=1e-12, atol=1e-12)
        assert np.allclose(dwu, gr["dwu"][i], rtol=1e-12, atol=1e-12)
        assert np.allclose(dwd, gr["dwd"][i], rtol=1e-12, atol=1e-12)


def test_planted_wrong_axis_is_caught(monkeypatch):
    """Quantising W_down's backward operand along F instead of H must break the brute-force match."""
    x, dy, lg, wg, wu, wd, k = _tiny(T=41)
    ref = _brute_mx(x, dy, lg, wg, wu, wd, k, False, True)
    orig = oracle.moe_oracle._qz

    def wrong(on, v, axis, **kw):
        if on and np.ndim(v) == 2 and np.shape(v) == wd[0].shape and axis == 0:
            axis = 1
        return orig(on, v, axis, **kw)
    monkeypatch.setattr(oracle.moe_oracle, "_qz", wrong)
    gr, _ = oracle.backward(dy, x, lg, wg, wu, wd, k, mode="fp8_bwd")
    assert not np.allclose(gr["dx"], ref[1], rtol=1e-9, atol=1e-9)
