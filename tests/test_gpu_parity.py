"""GPU parity: the HIP layer (through the C ABI) against the float64 oracle on the same seeded inputs.

Bar:
 * Routing (indices, counts, offsets, permutation, inverse): bit-exact.
 * Routing weights: within 1e-6 absolute.
 * y, dx, dlogits, dW_gate, dW_up, dW_down: relative Frobenius error within 1e-2 for bf16 and
   1e-5 for fp32.
 * Experts that receive no tokens: weight gradients exactly zero.
Full-size workloads are checked element by element against the full oracle: the whole-tensor bar
on every output, a per-row bound on y, dx and dlogits (5e-2 for bf16, against the row's norm or a
floor: 5 % of the typical row norm for y and dx, the typical row norm for dlogits), and the
whole-tensor bar on every expert's weight gradients.
"""
import numpy as np
import pytest
import torch

import oracle
from mixture_experts_layer_32_amd import inputs
from gpu_util import OUTS, ROW_TOL, TOL, run_layer
from mixture_experts_layer_32_amd.layer import MoELayer

pytestmark = pytest.mark.gpu


def check_routing(cfg, L, rt):
    r = oracle.route(L["logits"], cfg.k, cfg.e0, cfg.el)
    assert np.array_equal(rt["idx"], r["idx"]), "expert indices differ"
    assert np.array_equal(rt["counts"], r["counts"]), "expert counts differ"
    assert np.array_equal(rt["offsets"], r["offsets"]), "expert offsets differ"
    assert np.array_equal(rt["perm"], r["perm"]), "permutation differs"
    assert np.array_equal(rt["pair_pos"], r["pair_pos"]), "inverse permutation differs"
    assert np.max(np.abs(rt["weight"] - r["w"])) <= 1e-6
    return r


def oracle_full(cfg, L, mode="bf16"):
    """The float64 oracle's outputs; in the fp8 modes it quantises at the kernels' points (mode=...)."""
    args = dict(x=L["x"], logits=L["logits"], wg=L["wg"], wu=L["wu"], wd=L["wd"], k=cfg.k, e0=cfg.e0,
                e_local=cfg.el, mode=None if mode in ("fp32", "bf16") else mode)
    y, _ = oracle.forward(**args)
    g, _ = oracle.backward(dy=L["dy"], **args)
    return dict(y=y, dx=g["dx"], dlogits=g["dlogits"], dwg=g["dwg"], dwu=g["dwu"], dwd=g["dwd"])


def custom(name, mode="bf16", **kw):
    cfg, L = inputs.custom_layer(dtype=mode, **kw)
    return pytest.param(cfg.with_(name=name), L, mode, id=name)


SMALL = [
    pytest.param(inputs.CONFIGS["tiny"], None, "fp32", id="tiny_fp32"),
    pytest.param(inputs.CONFIGS["tiny"].with_(dtype="bf16"), None, "bf16", id="tiny_bf16"),
    custom("ragged_T333", T=333, H=512, F=256, E=16, k=4, seed=11),
    custom("ragged_fp32", mode="fp32", T=397, H=256, F=384, E=8, k=3, seed=12),
    # F = 384: the last N-tile of the down weight gradient holds 128 columns; ~337 pairs per expert
    # give every expert a full and a half M-tile
    custom("ragged_F384", T=900, H=512, F=384, E=8, k=3, seed=27),
    custom("k1", T=200, H=256, F=128, E=4, k=1, seed=13),
    custom("k_equals_E", T=96, H=256, F=128, E=4, k=4, seed=14),
    custom("single_token", T=1, H=256, F=128, E=8, k=2, seed=15),
    custom("zipf_empty_experts", T=300, H=256, F=256, E=32, k=2, zipf_s=3.0, seed=16),
    custom("expert_share", T=400, H=256, F=128, E=16, k=4, E_local=5, e0=3, seed=17),
    custom("expert_share_fp32", mode="fp32", T=250, H=256, F=128, E=12, k=3, E_local=4, e0=8, seed=18),
    custom("many_experts_k32", T=130, H=256, F=128, E=512, k=32, seed=19),
    # shares of at most a quarter of the experts: the backward runs two GEMMs per launch
    custom("share_quarter", T=700, H=512, F=384, E=32, k=4, E_local=8, e0=12, seed=25),
    custom("share_with_empty_experts", T=500, H=256, F=256, E=64, k=2, E_local=12, e0=14, zipf_s=0.3, seed=26),
    # several tokens per combine wavefront whose slot lanes lie past E (dlogits) and past the row's
    # chunks (H = 256): cross-lane reads from lanes outside a narrower loop's exec mask
    custom("share_small_E_k8", T=411, H=512, F=128, E=18, k=8, E_local=2, e0=16, zipf_s=1.1, seed=28),
    custom("share_k16_H256", T=300, H=256, F=128, E=40, k=16, E_local=8, e0=4, seed=29),
    custom("share_k16_H256_fp32", mode="fp32", T=300, H=256, F=128, E=40, k=16, E_local=8, e0=4, seed=29),
    custom("wide_H4096_F1536", T=130, H=4096, F=1536, E=4, k=2, seed=20),
]


@pytest.mark.parametrize("cfg,L,mode", SMALL)
def test_small_layer_parity(cfg, L, mode):
    if L is None:
        L = inputs.make_layer(cfg)
    print(f"case {cfg.name} mode={mode} T={cfg.T} H={cfg.H} F={cfg.F} E={cfg.E} k={cfg.k}", flush=True)
    got = run_layer(cfg, L, mode)
    r = check_routing(cfg, L, got["routing"])
    ref = oracle_full(cfg, L)
    errs = {n: oracle.rel_frobenius(got[n], ref[n]) for n in OUTS}
    print(cfg.name, {n: f"{v:.2e}" for n, v in errs.items()}, flush=True)
    for n in OUTS:
        assert errs[n] <= TOL[mode], (n, errs[n])
    empty = np.nonzero(r["counts"] == 0)[0]
    for e in empty:
        for n in ("dwg", "dwu", "dwd"):
            assert not np.any(got[n][e]), (n, e)
    if cfg.name == "zipf_empty_experts":
        assert empty.size > 0
    if cfg.el < cfg.E:                                   # tokens with no local pair: exact zeros
        none = np.nonzero(np.all(r["pair_pos"].reshape(cfg.T, cfg.k) < 0, axis=1))[0]
        assert not np.any(got["y"][none]) and not np.any(got["dx"][none])


@pytest.mark.parametrize("mode", ["bf16", "mxfp8", "fp8", "fp32"])
def test_share_with_no_local_pairs(mode):
    """An expert share that no token routes to (P = 0): every output is written, and exactly zero,
    whatever the workspace held (poisoned with NaN bit patterns)."""
    print(f"case share with no local pairs mode={mode}", flush=True)
    cfg, L = inputs.custom_layer(T=500, H=256, F=128, E=64, k=2, E_local=4, e0=60, zipf_s=5.0, seed=30,
                                 dtype="fp32" if mode == "fp32" else "bf16")
    got = run_layer(cfg, L, mode, poison=True)
    r = check_routing(cfg, L, got["routing"])
    assert r["counts"].sum() == 0
    for n in OUTS:
        assert not np.any(got[n]), n


def test_expert_shares_add_up_on_gpu():
    cfg, L = inputs.custom_layer(T=256, H=256, F=128, E=8, k=2, dtype="bf16", seed=21)
    full = run_layer(cfg, L)
    acc = {n: 0.0 for n in ("y", "dx", "dlogits")}
    for e0 in range(0, 8, 4):
        sc = cfg.with_(E_local=4, e0=e0)
        Ls = dict(L, wg=L["wg"][e0:e0 + 4], wu=L["wu"][e0:e0 + 4], wd=L["wd"][e0:e0 + 4])
        part = run_layer(sc, Ls)
        for n in acc:
            acc[n] = acc[n] + part[n]
        for n in ("dwg", "dwu", "dwd"):
            assert np.array_equal(part[n], full[n][e0:e0 + 4]), n
    for n in acc:
        assert oracle.rel_frobenius(acc[n], full[n]) <= 1e-2, n


def test_deterministic_and_poison_independent():
    cfg, L = inputs.custom_layer(T=300, H=512, F=256, E=16, k=4, dtype="bf16", seed=22)
    a = run_layer(cfg, L)
    b = run_layer(cfg, L, poison=True)
    for n in OUTS:
        assert a[n].tobytes() == b[n].tobytes(), n


# ------------------------------------------------------------------------------ full-size workloads

def row_errors(got, ref, floor_frac=0.05):
    """Per-row relative error ||got_t - ref_t|| / max(||ref_t||, floor), with floor = floor_frac times
    the root-mean-square norm of the reference's rows: a row whose reference is far below the typical
    row norm (a dlogits row whose router gradients nearly cancel) is judged against that floor."""
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    d = np.linalg.norm(got - ref, axis=1)
    n = np.linalg.norm(ref, axis=1)
    rms = np.sqrt(np.mean(n ** 2))
    return d / np.maximum(n, floor_frac * rms)


def full_check(cfg, L, got, mode="bf16"):
    """Every output element against the full float64 oracle: the whole-tensor bar, a per-row bound on
    y, dx and dlogits, and the whole-tensor bar on every expert's dW_gate, dW_up and dW_down."""
    r = check_routing(cfg, L, got["routing"])
    print(f"case {cfg.name}: float64 oracle on the host", flush=True)
    ref = oracle_full(cfg, L, mode)
    errs = {n: oracle.rel_frobenius(got[n], ref[n]) for n in OUTS}
    # A dlogits row is w_j (g_j - sum_i w_i g_i) over the token's chosen experts, with g_j = <dY_t, o_tj>:
    # its size follows how far the router gradients cancel (in an expert share a row can hang on one
    # g), while the rounding error of each g follows |dY_t| |o_tj|. Its rows are therefore judged
    # against at least the typical row norm; y and dx rows against 5 % of it.
    rows = {n: row_errors(got[n], ref[n], 1.0 if n == "dlogits" else 0.05) for n in ("y", "dx", "dlogits")}
    per_e = {n: np.array([oracle.rel_frobenius(got[n][e], ref[n][e]) if r["counts"][e] else 0.0
                          for e in range(cfg.el)]) for n in ("dwg", "dwu", "dwd")}
    print(cfg.name, "counts min/max", r["counts"].min(), r["counts"].max(),
          {n: f"{v:.2e}" for n, v in errs.items()},
          {f"{n} rows max/p99.9": f"{v.max():.2e}/{np.percentile(v, 99.9):.2e}" for n, v in rows.items()},
          {f"{n} experts max": f"{v.max():.2e}" for n, v in per_e.items()}, flush=True)
    for n in OUTS:
        assert errs[n] <= TOL[mode], (n, errs[n])
        assert np.all(np.isfinite(got[n])), n
    for n, v in rows.items():
        worst = int(np.argmax(v))
        assert v[worst] <= ROW_TOL[mode], (n, "row", worst, v[worst])
    for n, v in per_e.items():
        worst = int(np.argmax(v))
        assert v[worst] <= TOL[mode], (n, "expert", worst, v[worst])
    for e in np.nonzero(r["counts"] == 0)[0]:
        for n in ("dwg", "dwu", "dwd"):
            assert not np.any(got[n][e]), (n, e)
    # rows of tokens with no pair on the computed experts are exactly zero
    none = np.nonzero(np.all(r["pair_pos"].reshape(cfg.T, cfg.k) < 0, axis=1))[0]
    for n in ("y", "dx", "dlogits"):
        assert not np.any(got[n][none]), n


@pytest.mark.slow
@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["qwen3_30b_a3b", "qwen3_30b_a3b_ep16", "qwen3_235b_a22b_zipf"])
def test_full_size_every_output(name):
    """The full-size workloads, every row of y, dx and dlogits and every expert's weight gradients
    compared with the float64 oracle (no sampling)."""
    cfg = inputs.CONFIGS[name]
    print(f"case {name}: generating inputs", flush=True)
    L = inputs.make_layer(cfg)
    print(f"case {name}: running fwd+bwd on the GPU", flush=True)
    got = run_layer(cfg, L)
    torch.cuda.empty_cache()
    full_check(cfg, L, got)


# rows per expert at the edges of the 128-row (half) and 256-row tiles, and an empty expert
TILE_COUNTS = [128, 129, 255, 256, 257, 1, 0, 127, 384, 385]


@pytest.mark.parametrize("mode", ["bf16", "mxfp8", "fp8_bwd", "fp8"])
def test_tile_boundary_counts(mode):
    """k = 1 routing forced onto chosen experts (the chosen logit is 6 above the others), so that the
    expert segments end exactly at, just before and just after the tile edges: half tiles, whole
    tiles, one-row tails and an empty expert."""
    E, T = len(TILE_COUNTS), sum(TILE_COUNTS)
    cfg, L = inputs.custom_layer(T=T, H=256, F=128, E=E, k=1, seed=23)
    rng = np.random.default_rng(24)
    assign = np.repeat(np.arange(E), TILE_COUNTS)
    rng.shuffle(assign)
    lg = (0.1 * rng.standard_normal((T, E))).astype(np.float32)
    lg[np.arange(T), assign] += np.float32(6.0)
    L = dict(L, logits=lg)
    print(f"case tile_boundary_counts mode={mode} counts={TILE_COUNTS}", flush=True)
    got = run_layer(cfg, L, mode)
    r = check_routing(cfg, L, got["routing"])
    assert list(r["counts"]) == TILE_COUNTS
    args = dict(x=L["x"], logits=lg, wg=L["wg"], wu=L["wu"], wd=L["wd"], k=1, mode=None if mode == "bf16" else mode)
    y, _ = oracle.forward(**args)
    g, _ = oracle.backward(dy=L["dy"], **args)
    ref = dict(y=y, dx=g["dx"], dlogits=g["dlogits"], dwg=g["dwg"], dwu=g["dwu"], dwd=g["dwd"])
    errs = {n: oracle.rel_frobenius(got[n], ref[n]) for n in OUTS if n != "dlogits"}
    print("tile_boundary_counts", mode, {n: f"{v:.2e}" for n, v in errs.items()}, flush=True)
    for n, v in errs.items():
        assert v <= TOL[mode], (n, v)
    # k = 1: the weights are 1 and dlogits is exactly zero
    assert not np.any(got["dlogits"])
    for n in ("dwg", "dwu", "dwd"):
        assert not np.any(got[n][TILE_COUNTS.index(0)]), n


def test_wgrad_xcd_split_balances_a_skewed_load():
    """The weight-gradient tile lists are cut into 8 per-XCD ranges of equal estimated cost when equal
    tile counts would be out of balance (a Zipf-like skew here). White-box: the ranges sit in the
    backward workspace's scheduler slots 2 (down) and 3 (gate/up), 9 boundaries each."""
    H, F, E, k = 1024, 512, 32, 2
    cfg, L = inputs.custom_layer(T=3000, H=H, F=F, E=E, k=k, zipf_s=2.5, seed=77)
    print("case wgrad_xcd_split zipf_s=2.5", flush=True)
    got = run_layer(cfg, L, "bf16", keep_layer=True)
    layer = got["_layer"]
    ws = layer.ws[:8 * 16 * 4].cpu().numpy().view(np.int32).reshape(8, 16)
    counts = got["routing"]["counts"].astype(np.int64)
    u = -(-counts // 64) + 2                                    # K-tiles per tile, plus its fixed cost
    for slot, tpe in ((2, (H // 256) * -(-F // 256)), (3, (2 * F // 256) * (H // 256))):
        b = ws[slot, :9]
        assert b[0] == 0 and b[8] == E * tpe and np.all(np.diff(b) >= 0), b
        tile_cost = np.repeat(u, tpe)
        cost = np.array([tile_cost[b[x]:b[x + 1]].sum() for x in range(8)])
        per = -(-E * tpe // 8)
        even = np.array([tile_cost[x * per:(x + 1) * per].sum() for x in range(8)])
        assert even.max() > 1.1 * even.mean()                   # the skew defeats equal counts
        assert cost.max() <= cost.sum() / 8 + tile_cost.max(), (cost, b)
        assert cost.max() < even.max()


@pytest.mark.slow
@pytest.mark.timeout(600)
@pytest.mark.parametrize("mode", ["bf16", "mxfp8"])
def test_element_offsets_beyond_32_bits(mode):
    """320 k routed pairs of H = 7168 (2.3e9 elements in the per-pair buffers the down GEMM writes, the
    dgrad of x writes and both combines read): y, dx and dlogits rows of the tokens whose pairs sit
    at the highest positions, and of a few others, against the oracle computed from those tokens'
    own pairs."""
    print(f"case offsets beyond 32 bits: T=160000 H=7168 F=2048 E=4 k=2 mode={mode}", flush=True)
    cfg, L = inputs.custom_layer(T=160000, H=7168, F=2048, E=4, k=2, seed=32)
    dt = torch.bfloat16
    dev = lambda a, t=dt: torch.from_numpy(np.ascontiguousarray(a)).to("cuda").to(t)
    x, dy, lg = dev(L["x"]), dev(L["dy"]), dev(L["logits"], torch.float32)
    wg, wu, wd = dev(L["wg"]), dev(L["wu"]), dev(L["wd"])
    layer = MoELayer(cfg.T, cfg.H, cfg.F, cfg.E, cfg.k, mode)
    y = layer.forward(x, lg, wg, wu, wd)
    g = layer.backward(dy, x, wg, wu, wd)
    torch.cuda.synchronize()
    rt = layer.routing()
    pp = rt["pair_pos"].numpy().reshape(cfg.T, cfg.k)
    assert int(rt["offsets"][-1]) * cfg.H >= 2 ** 31
    top = np.argsort(-pp.max(axis=1))[:8]                  # pairs at the highest positions
    rest = np.random.default_rng(33).choice(cfg.T, 8, replace=False)
    toks = np.unique(np.concatenate([top, rest]))
    ti = torch.from_numpy(toks).to("cuda")
    got = dict(y=y[ti].float().cpu().numpy(), dx=g["dx"][ti].float().cpu().numpy(),
               dlogits=g["dlogits"][ti].cpu().numpy())
    ref = oracle.token_rows(toks, L["dy"], L["x"], L["logits"], L["wg"], L["wu"], L["wd"], cfg.k,
                            mode=None if mode == "bf16" else mode)
    for n in ("y", "dx", "dlogits"):
        ref_n = ref[n]
        e = oracle.rel_frobenius(got[n], ref_n)
        worst = float(np.max(row_errors(got[n], ref_n)))
        print(n, f"{e:.2e} worst row {worst:.2e}", flush=True)
        assert e <= TOL[mode] and worst <= ROW_TOL[mode], (n, e, worst)
