"""Pins of the oracle's blockwise FP8 emulation and the "fp8" precision mode (CPU only).

The quantiser is checked against things it does not share code with:
 * the scale exponent by a linear search for the smallest power of two that holds the block;
 * elements by torch's float8_e4m3fn cast, and by brute-force nearest search over the 254 finite
   E4M3 values;
 * the tile structure of the weights by orientation and per-tile scaling invariants.
The layer's data flow in this mode is checked against a per-pair brute force whose quantisers are
built from those two independent pieces.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import mx


def _search_exponent(amax):
    """Smallest integer s in [-127, 127] with amax <= 448 * 2^s, by linear search (-127 for 0)."""
    if amax == 0:
        return -127
    for s in range(-127, 128):
        if amax <= 448.0 * 2.0 ** s:
            return s
    return 127


def _torch_e4m3(v):
    return torch.from_numpy(np.asarray(v, np.float32)).to(torch.float8_e4m3fn).to(torch.float64).numpy()


def _torch_blocks(v, axis, block=128):
    """Round trip along `axis` in zero-padded blocks of `block`: searched scale, torch's cast."""
    x = np.moveaxis(np.asarray(v, np.float64), axis, -1)
    out = np.empty_like(x)
    flat_in, flat_out = x.reshape(-1, x.shape[-1]), out.reshape(-1, x.shape[-1])
    for r in range(flat_in.shape[0]):
        for b0 in range(0, flat_in.shape[1], block):
            blk = flat_in[r, b0:b0 + block]
            sc = 2.0 ** _search_exponent(np.abs(blk).max())
            flat_out[r, b0:b0 + block] = _torch_e4m3(blk / sc) * sc
    return np.moveaxis(out, -1, axis)


def _torch_tiles(w, tile=128):
    w = np.asarray(w, np.float64)
    out = np.empty_like(w)
    for r0 in range(0, w.shape[0], tile):
        for c0 in range(0, w.shape[1], tile):
            t = w[r0:r0 + tile, c0:c0 + tile]
            sc = 2.0 ** _search_exponent(np.abs(t).max())
            out[r0:r0 + tile, c0:c0 + tile] = _torch_e4m3(t / sc) * sc
    return out


# ---------------------------------------------------------------------------------------------
# the scale rule and the quantisers

def test_ceil_scale_matches_linear_search():
    rng = np.random.default_rng(3)
    amax = np.concatenate([np.ldexp(rng.uniform(1, 2, 400), rng.integers(-120, 120, 400)),
                           np.ldexp(448.0, np.arange(-20, 20)), np.ldexp(1.75, np.arange(-20, 20)),
                           [0.0, 1e-45, 3e38, 224.0, 224.00001, 447.99999, 448.00001]])
    got = mx.ceil_scale_exponent(amax)
    ref = np.array([_search_exponent(a) for a in amax])
    assert np.array_equal(got, ref)


def test_ceil_scale_boundaries():
    assert mx.ceil_scale_exponent(448.0) == 0
    assert mx.ceil_scale_exponent(np.nextafter(448.0, 1e9)) == 1
    assert mx.ceil_scale_exponent(224.0) == -1
    assert mx.ceil_scale_exponent(0.0) == -127
    assert mx.ceil_scale_exponent(2.0 ** -140) == -127      # clamped from below; still holds the block
    assert mx.ceil_scale_exponent(1.0) == -8                 # 1 <= 448 / 256, and 1 > 448 / 512


def test_block_quantize_never_saturates_and_rounds_to_nearest():
    rng = np.random.default_rng(5)
    v = rng.standard_normal((40, 128)) * np.ldexp(1.0, rng.integers(-30, 30, (40, 1)))
    v[3, 17] = 0.0
    v[7] = 0.0
    deq, el, s = mx.fp8_block_quantize(v, axis=1, return_parts=True)
    table = np.sort(mx.e4m3_table())
    assert np.abs(el).max() <= 448.0
    for r in range(v.shape[0]):
        sc = 2.0 ** s[r, 0]
        assert s[r, 0] == _search_exponent(np.abs(v[r]).max())
        d = np.abs(table[None, :] - (v[r] / sc)[:, None])
        best = table[np.argmin(d, axis=1)]
        # nearest value; at an exact tie either neighbour is nearest, torch's cast decides below
        assert np.allclose(np.abs(best - v[r] / sc), np.abs(el[r] - v[r] / sc), rtol=0, atol=0)
        if np.abs(v[r]).max() > 0:                            # the block's largest element: 3-bit mantissa
            i = np.argmax(np.abs(v[r]))
            assert abs(deq[r, i] - v[r, i]) <= abs(v[r, i]) * 2.0 ** -4
    assert np.array_equal(deq[7], np.zeros(128))


@pytest.mark.parametrize("axis", [0, 1])
def test_block_quantize_matches_torch_quantiser_with_ragged_tail(axis):
    rng = np.random.default_rng(11)
    v = rng.standard_normal((300, 9) if axis == 0 else (9, 300)).astype(np.float32).astype(np.float64)
    assert np.array_equal(mx.fp8_block_quantize(v, axis=axis), _torch_blocks(v, axis))


def test_block_quantize_blocks_are_independent():
    rng = np.random.default_rng(12)
    v = rng.standard_normal(300)
    whole = mx.fp8_block_quantize(v)
    parts = np.concatenate([mx.fp8_block_quantize(v[:128]), mx.fp8_block_quantize(v[128:256]),
                            mx.fp8_block_quantize(v[256:])])
    assert np.array_equal(whole, parts)


def test_tile_quantize_matches_torch_and_is_orientation_free():
    rng = np.random.default_rng(13)
    w = (rng.standard_normal((256, 384)) / 16).astype(np.float32).astype(np.float64)
    q = mx.fp8_tile_quantize(w)
    assert np.array_equal(q, _torch_tiles(w))
    assert np.array_equal(mx.fp8_tile_quantize(w.T), q.T)


def test_tile_quantize_scales_per_tile():
    rng = np.random.default_rng(14)
    w = rng.standard_normal((256, 256))
    q0 = mx.fp8_tile_quantize(w)
    w2 = w.copy()
    w2[128:, :128] *= 2.0 ** 10                       # one tile scaled by a power of two
    q2 = mx.fp8_tile_quantize(w2)
    assert np.array_equal(q2[128:, :128], q0[128:, :128] * 2.0 ** 10)
    mask = np.ones_like(w, bool)
    mask[128:, :128] = False
    assert np.array_equal(q2[mask], q0[mask])
    w3 = w.copy()
    w3[0, 0] = 1e4                                    # an outlier coarsens its own tile only
    q3 = mx.fp8_tile_quantize(w3)
    assert np.array_equal(q3[:, 128:], q0[:, 128:])
    assert np.array_equal(q3[128:], q0[128:])
    assert not np.array_equal(q3[1:128, 1:128], q0[1:128, 1:128])


# ---------------------------------------------------------------------------------------------
# the layer in the "fp8" mode

def _layer(seed=7, T=300, H=256, F=192, E=4, k=2):
    rng = np.random.default_rng(seed)
    f32 = lambda a: a.astype(np.float32).astype(np.float64)
    x = f32(rng.standard_normal((T, H)))
    dy = f32(rng.standard_normal((T, H)))
    lg = f32(rng.standard_normal((T, E)))
    wg = f32(rng.standard_normal((E, F, H)) / 16)
    wu = f32(rng.standard_normal((E, F, H)) / 16)
    wd = f32(rng.standard_normal((E, H, F)) / 14)
    return x, dy, lg, wg, wu, wd, k


def _brute_fp8(x, dy, lg, wg, wu, wd, k):
    """Per token and slot loops with the searched-scale, torch-cast quantisers: 1 x 128 blocks along
    each GEMM's contraction axis for activations, 128 x 128 tiles for weights; weight-gradient
    operands blocked along each expert's pairs in ascending pair order (token-major, then slot)."""
    T, H = x.shape
    E, F, _ = wg.shape
    sg = lambda z: 1 / (1 + np.exp(-z))
    QA = _torch_blocks
    qwg = [_torch_tiles(wg[e]) for e in range(E)]
    qwu = [_torch_tiles(wu[e]) for e in range(E)]
    qwd = [_torch_tiles(wd[e]) for e in range(E)]
    y = np.zeros((T, H))
    dx = np.zeros((T, H))
    g = np.zeros((T, k))
    rows = {e: [] for e in range(E)}
    for t in range(T):
        order = sorted(range(E), key=lambda e: (-lg[t, e], e))[:k]
        z = np.exp(lg[t, order] - lg[t, order].max())
        w = z / z.sum()
        xr = QA(x[t:t + 1], 1)
        dyr = QA(dy[t:t + 1], 1)
        for j, e in enumerate(order):
            a = xr @ qwg[e].T
            b = xr @ qwu[e].T
            h = a * sg(a) * b
            y[t] += (QA(w[j] * h, 1) @ qwd[e].T)[0]
            u = dyr @ qwd[e]
            g[t, j] = np.sum(u * h)
            dh = w[j] * u
            da = dh * b * sg(a) * (1 + a * (1 - sg(a)))
            db = dh * a * sg(a)
            dx[t] += (QA(da, 1) @ qwg[e] + QA(db, 1) @ qwu[e])[0]
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
        dwd[e] = QA(dy[ts], 0).T @ QA(HW, 0)
        dwg[e] = QA(DA, 0).T @ QA(x[ts], 0)
        dwu[e] = QA(DB, 0).T @ QA(x[ts], 0)
    return y, dx, g, dwg, dwu, dwd, rows


def test_fp8_mode_matches_brute_force():
    L = _layer()
    ref = _brute_fp8(*L)
    assert max(len(r) for r in ref[6].values()) > 128     # several 128-pair blocks per expert
    x, dy, lg, wg, wu, wd, k = L
    y, _ = oracle.forward(x, lg, wg, wu, wd, k, mode="fp8")
    gr, _ = oracle.backward(dy, x, lg, wg, wu, wd, k, mode="fp8")
    for got, want in ((y, ref[0]), (gr["dx"], ref[1]), (gr["g"], ref[2]), (gr["dwg"], ref[3]), (gr["dwu"], ref[4]),
                      (gr["dwd"], ref[5])):
        assert np.allclose(got, want, rtol=1e-9, atol=1e-9)


def test_fp8_mode_stays_close_to_exact_and_differs_from_mxfp8():
    x, dy, lg, wg, wu, wd, k = _layer(T=160)
    y0, _ = oracle.forward(x, lg, wg, wu, wd, k)
    g0, _ = oracle.backward(dy, x, lg, wg, wu, wd, k)
    y1, _ = oracle.forward(x, lg, wg, wu, wd, k, mode="fp8")
    g1, _ = oracle.backward(dy, x, lg, wg, wu, wd, k, mode="fp8")
    y2, _ = oracle.forward(x, lg, wg, wu, wd, k, mode="mxfp8")
    assert 1e-3 < oracle.rel_frobenius(y1, y0) < 0.1
    assert oracle.rel_frobenius(y1, y2) > 1e-3
    for n in ("dx", "dlogits", "dwg", "dwu", "dwd"):
        assert 1e-3 < oracle.rel_frobenius(g1[n], g0[n]) < 0.12, n


def test_fp8_row_and_expert_helpers_agree_with_full_passes():
    x, dy, lg, wg, wu, wd, k = _layer(T=200)
    y, r = oracle.forward(x, lg, wg, wu, wd, k, mode="fp8")
    gr, _ = oracle.backward(dy, x, lg, wg, wu, wd, k, mode="fp8")
    toks = [0, 7, 133, 199]
    rows = oracle.token_rows(toks, dy, x, lg, wg, wu, wd, k, mode="fp8")
    for n, full in (("y", y), ("dx", gr["dx"]), ("dlogits", gr["dlogits"])):
        assert np.allclose(rows[n], full[toks], rtol=1e-12, atol=1e-12), n
    for i in range(4):
        dwg, dwu, dwd = oracle.expert_grads(i, dy, x, lg, wg[i], wu[i], wd[i], k, r=r, mode="fp8")
        assert np.allclose(dwg, gr["dwg"][i], rtol=1e-12, atol=1e-12)
        assert np.allclose(dwu, gr["dwu"][i], rtol=1e-12, atol=1e-12)
        assert np.allclose(dwd, gr["dwd"][i], rtol=1e-12, atol=1e-12)


def test_planted_row_blocks_for_weights_are_caught(monkeypatch):
    """Quantising a weight in 1 x 128 row blocks instead of 128 x 128 tiles must break the match."""
    L = _layer(T=120)
    ref = _brute_fp8(*L)
    x, dy, lg, wg, wu, wd, k = L
    orig = oracle.moe_oracle._qz

    def wrong(kind, v, axis, weight=False):
        return orig(kind, v, axis, weight=False)
    monkeypatch.setattr(oracle.moe_oracle, "_qz", wrong)
    y, _ = oracle.forward(x, lg, wg, wu, wd, k, mode="fp8")
    assert not np.allclose(y, ref[0], rtol=1e-9, atol=1e-9)
