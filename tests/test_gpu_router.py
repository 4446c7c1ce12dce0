"""GPU parity of the router projection in front of the layer (moe_router_fwd, moe_router_bwd)
against the float64 oracle (oracle.router_forward, oracle.router_backward).

Bar (relative Frobenius error per output, as for the layer):
 * logits <= 1e-5. Products of bf16 values are exact in fp32, and the fp32 sums (MFMA blocks over H,
   two interleaved chains; beyond 256 experts H-slices, then at most 4 slice partials in a fixed
   order) stay within a few 2^-24 sqrt(H) of the float64 values relative to the row's scale: about
   4e-6 at H = 4096.
 * dW_r and the router's part of dx <= 1e-2 (the bf16 bar): the backward multiplies a bf16 copy of
   dlogits (relative rounding 2^-9) and rounds its outputs to bf16 once.
 * Bitwise reproducible across calls.
 * The fp32 test mode (fp32 tensors, plain fp32 sums): every output <= 1e-5.
The composition test runs x, W_r -> router -> layer -> router backward on the GPU and compares the
total dx and dW_r with the oracle's chain on the same fp32 logits (so that both route alike).
Up to 256 experts moe_router_fwd runs the fused forward's projection (one pass over H per 64 tokens),
so its logits are bitwise those moe_fwd_router routes on; beyond, split-H partial sums.
"""
import numpy as np
import pytest
import torch

import oracle
from mixture_experts_layer_32_amd import inputs
from mixture_experts_layer_32_amd.layer import MoELayer
from gpu_util import to_dev, run_layer

pytestmark = pytest.mark.gpu

TOL_LOGITS = 1e-5
TOL_BWD = 1e-2
TOL_FP32 = 1e-5   # the fp32 test mode: plain fp32 sums of at most 16384 terms


def sparse_dlogits(T, E, k, seed):
    """k nonzero entries per row, like the layer's dlogits."""
    rng = np.random.default_rng(seed)
    dl = np.zeros((T, E), np.float32)
    for t in range(T):
        dl[t, rng.choice(E, size=min(k, E), replace=False)] = rng.standard_normal(min(k, E)).astype(np.float32)
    return dl


CASES = [
    ("basic", dict(T=256, H=256, E=8, k=2), "bf16"),
    ("ragged_T300_E40", dict(T=300, H=256, E=40, k=3), "bf16"),
    ("E128_T513_H512", dict(T=513, H=512, E=128, k=8), "bf16"),
    ("E200_H768", dict(T=1000, H=768, E=200, k=4), "bf16"),
    ("E512_T70", dict(T=70, H=256, E=512, k=8), "bf16"),
    ("single_token", dict(T=1, H=256, E=8, k=2), "bf16"),
    ("wide_H4096", dict(T=130, H=4096, E=64, k=4), "bf16"),
    ("mxfp8_mode", dict(T=300, H=512, E=40, k=3), "mxfp8"),
    ("fp32_mode", dict(T=300, H=256, E=40, k=3), "fp32"),
    ("fp32_mode_E200", dict(T=517, H=512, E=200, k=4), "fp32"),
]


def router_inputs(T, H, E, k, seed, dtype="bf16"):
    cfg, L = inputs.custom_layer(T=T, H=H, F=128, E=E, k=k, seed=seed, dtype=dtype)
    return cfg, L["x"], inputs.router_weight(cfg)


def _router_sweep_case(i):
    rng = np.random.default_rng(7000 + i)
    E = int(rng.integers(1, 513))
    shape = dict(T=int(rng.integers(1, 1500)), H=int(rng.choice([256, 512, 768, 1024, 2048])), E=E,
                 k=int(rng.integers(1, min(32, E) + 1)))
    return (f"sweep{i}", shape, ("bf16", "bf16", "mxfp8", "fp32")[i % 4])


CASES += [_router_sweep_case(i) for i in range(16)]


@pytest.mark.parametrize("name,shape,mode", CASES, ids=[c[0] for c in CASES])
def test_router_parity(name, shape, mode):
    print(f"case router {name} mode={mode} {shape}", flush=True)
    f32 = mode == "fp32"
    dt = torch.float32 if f32 else torch.bfloat16
    tol_bwd = TOL_FP32 if f32 else TOL_BWD
    cfg, x, wr = router_inputs(**shape, seed=51, dtype="fp32" if f32 else "bf16")
    T, H, E = cfg.T, cfg.H, cfg.E
    layer = MoELayer(T, H, 128, E, cfg.k, mode)
    xd, wrd = to_dev(x, dt), to_dev(wr, dt)
    lg = layer.router_forward(xd, wrd)
    torch.cuda.synchronize()
    ref = oracle.router_forward(x, wr)
    e_fwd = oracle.rel_frobenius(lg.cpu().numpy(), ref)
    for dense in (False, True):
        dl = np.random.default_rng(52).standard_normal((T, E)).astype(np.float32) if dense \
            else sparse_dlogits(T, E, cfg.k, 53)
        dwr_ref, dxr_ref = oracle.router_backward(dl, x, wr)
        dx0 = np.zeros((T, H), np.float32)
        dx = to_dev(dx0, dt)
        dwr = layer.router_backward(xd, wrd, to_dev(dl, torch.float32), dx)
        torch.cuda.synchronize()
        e_dw = oracle.rel_frobenius(dwr.float().cpu().numpy(), dwr_ref)
        e_dx = oracle.rel_frobenius(dx.float().cpu().numpy(), dxr_ref)
        # dx is accumulated into: start from a nonzero dx of the same scale
        dx1 = (np.random.default_rng(54).standard_normal((T, H)) * np.sqrt(np.mean(dxr_ref ** 2))).astype(np.float32)
        if not f32:
            dx1 = inputs.round_to_bf16(dx1)
        dxt = to_dev(dx1, dt)
        layer.router_backward(xd, wrd, to_dev(dl, torch.float32), dxt)
        torch.cuda.synchronize()
        e_acc = oracle.rel_frobenius(dxt.float().cpu().numpy(), dx1.astype(np.float64) + dxr_ref)
        print(name, "dense" if dense else "sparse", f"logits {e_fwd:.2e} dW_r {e_dw:.2e} dx {e_dx:.2e} "
              f"dx accumulated {e_acc:.2e}", flush=True)
        assert e_dw <= tol_bwd and e_dx <= tol_bwd and e_acc <= tol_bwd
    assert e_fwd <= TOL_LOGITS


def test_router_deterministic():
    print("case router determinism", flush=True)
    cfg, x, wr = router_inputs(T=700, H=512, E=96, k=4, seed=61)
    layer = MoELayer(cfg.T, cfg.H, 128, cfg.E, cfg.k, "bf16")
    xd, wrd = to_dev(x, torch.bfloat16), to_dev(wr, torch.bfloat16)
    dl = to_dev(sparse_dlogits(cfg.T, cfg.E, cfg.k, 62), torch.float32)
    outs = []
    ws = layer._router_ws()
    for rep in range(2):
        ws.fill_(0xFF if rep == 0 else 0x00)     # results must not depend on stale workspace bytes
        lg = layer.router_forward(xd, wrd)
        dx = torch.zeros(cfg.T, cfg.H, dtype=torch.bfloat16, device="cuda")
        dwr = layer.router_backward(xd, wrd, dl, dx)
        torch.cuda.synchronize()
        outs.append([t.cpu().numpy().tobytes() for t in (lg, dx.view(torch.int16), dwr.view(torch.int16))])
    assert outs[0] == outs[1]


@pytest.mark.parametrize("E", [96, 40, 37])
def test_router_backward_dlogits_alignment(E):
    """dlogits needs only 4-byte alignment: a copy at a 4-byte offset (and rows of E % 4 != 0 floats)
    takes the conversion's scalar loads, and must give the bits of the 16-byte-aligned call."""
    print(f"case router dlogits alignment E={E}", flush=True)
    cfg, x, wr = router_inputs(T=300, H=256, E=E, k=4, seed=63)
    layer = MoELayer(cfg.T, cfg.H, 128, cfg.E, cfg.k, "bf16")
    xd, wrd = to_dev(x, torch.bfloat16), to_dev(wr, torch.bfloat16)
    dl_np = sparse_dlogits(cfg.T, cfg.E, cfg.k, 64)
    dl = to_dev(dl_np, torch.float32)
    buf = torch.empty(cfg.T * cfg.E + 4, dtype=torch.float32, device="cuda")
    dl_off = buf[1:1 + cfg.T * cfg.E].view(cfg.T, cfg.E)
    dl_off.copy_(dl)
    assert dl_off.data_ptr() % 16 == 4
    outs = []
    for d in (dl, dl_off):
        dx = torch.zeros(cfg.T, cfg.H, dtype=torch.bfloat16, device="cuda")
        dwr = layer.router_backward(xd, wrd, d, dx)
        torch.cuda.synchronize()
        outs.append((dx.view(torch.int16).clone(), dwr.view(torch.int16).clone()))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
    dwr_ref, dxr_ref = oracle.router_backward(dl_np, x, wr)
    assert oracle.rel_frobenius(outs[0][1].view(torch.bfloat16).float().cpu().numpy(), dwr_ref) <= TOL_BWD


def test_router_then_layer_composition():
    """x, W_r -> logits -> layer forward/backward -> router backward, all on the GPU."""
    print("case router composition", flush=True)
    cfg, L = inputs.custom_layer(T=400, H=256, F=128, E=16, k=4, seed=71)
    wr = inputs.router_weight(cfg)
    layer = MoELayer(cfg.T, cfg.H, cfg.F, cfg.E, cfg.k, "bf16")
    xd, wrd = to_dev(L["x"], torch.bfloat16), to_dev(wr, torch.bfloat16)
    lg = layer.router_forward(xd, wrd)
    torch.cuda.synchronize()
    lg_np = lg.cpu().numpy()
    assert oracle.rel_frobenius(lg_np, oracle.router_forward(L["x"], wr)) <= TOL_LOGITS
    # the layer on the GPU's logits (both sides route on the same fp32 bits)
    L2 = dict(L, logits=lg_np)
    got = run_layer(cfg, L2, keep_layer=True)
    gl = got["_layer"]
    r = oracle.route(lg_np, cfg.k)
    assert np.array_equal(got["routing"]["idx"], r["idx"])
    dx = to_dev(got["dx"].astype(np.float32), torch.bfloat16)
    dwr = gl.router_backward(xd, wrd, to_dev(got["dlogits"].astype(np.float32), torch.float32), dx)
    torch.cuda.synchronize()
    args = dict(x=L["x"], logits=lg_np, wg=L["wg"], wu=L["wu"], wd=L["wd"], k=cfg.k)
    g, _ = oracle.backward(dy=L["dy"], **args)
    dwr_ref, dxr_ref = oracle.router_backward(g["dlogits"], L["x"], wr)
    e_dx = oracle.rel_frobenius(dx.float().cpu().numpy(), g["dx"] + dxr_ref)
    e_dw = oracle.rel_frobenius(dwr.float().cpu().numpy(), dwr_ref)
    print(f"composition dx {e_dx:.2e} dW_r {e_dw:.2e}", flush=True)
    assert e_dx <= TOL_BWD and e_dw <= TOL_BWD


@pytest.mark.slow
def test_router_full_size_sampled():
    """The benchmark shape (T=16384, H=2048, E=128): sampled logits rows, dx rows and dW_r rows."""
    cfg = inputs.CONFIGS["qwen3_30b_a3b"]
    print(f"case router full size {cfg.name}", flush=True)
    x, _, _ = inputs.make_tokens(cfg)
    wr = inputs.router_weight(cfg)
    layer = MoELayer(cfg.T, cfg.H, cfg.F, cfg.E, cfg.k, "bf16")
    xd, wrd = to_dev(x, torch.bfloat16), to_dev(wr, torch.bfloat16)
    lg = layer.router_forward(xd, wrd)
    dl = sparse_dlogits(cfg.T, cfg.E, cfg.k, 81)
    dx = torch.zeros(cfg.T, cfg.H, dtype=torch.bfloat16, device="cuda")
    dwr = layer.router_backward(xd, wrd, to_dev(dl, torch.float32), dx)
    torch.cuda.synchronize()
    rows = np.random.default_rng(82).choice(cfg.T, size=64, replace=False)
    experts = np.random.default_rng(83).choice(cfg.E, size=8, replace=False)
    e_l = oracle.rel_frobenius(lg.cpu().numpy()[rows], oracle.router_forward(x[rows], wr))
    e_x = oracle.rel_frobenius(dx.float().cpu().numpy()[rows], oracle.router_backward(dl[rows], x[rows], wr)[1])
    dw_ref = dl[:, experts].astype(np.float64).T @ x.astype(np.float64)
    e_w = oracle.rel_frobenius(dwr.float().cpu().numpy()[experts], dw_ref)
    print(f"full size: logits {e_l:.2e} dx {e_x:.2e} dW_r {e_w:.2e}", flush=True)
    assert e_l <= TOL_LOGITS and e_x <= TOL_BWD and e_w <= TOL_BWD


# ------------------------------------------------------------- router projection fused with routing
FUSED = [
    # name, T, H, F, E, k, E_local, e0, mode
    ("E8_k2", 256, 256, 128, 8, 2, None, 0, "bf16"),
    ("E128_k8_ragged", 777, 512, 256, 128, 8, None, 0, "bf16"),
    ("E160_k6_two_blocks", 300, 256, 128, 160, 6, None, 0, "bf16"),
    ("E256_k8", 200, 768, 128, 256, 8, None, 0, "bf16"),
    ("E128_share", 500, 256, 128, 128, 8, 16, 32, "bf16"),
    ("E64_k1", 129, 256, 128, 64, 1, None, 0, "bf16"),
    ("E128_mxfp8", 300, 512, 256, 128, 8, None, 0, "mxfp8"),
]


def _fused_sweep_case(i):
    rng = np.random.default_rng(8000 + i)
    E = int(rng.integers(2, 257))
    k = int(rng.integers(1, min(8, E) + 1))
    share = rng.random() < 0.3
    el = int(rng.integers(1, E + 1)) if share else None
    e0 = int(rng.integers(0, E - el + 1)) if share else 0
    return (f"sweep{i}", int(rng.integers(1, 1200)), int(rng.choice([256, 512, 1024])), 128, E, k, el, e0,
            ("bf16", "mxfp8", "fp8_bwd", "fp8")[i % 4])


FUSED += [_fused_sweep_case(i) for i in range(12)]


@pytest.mark.parametrize("name,T,H,F,E,k,el,e0,mode", FUSED, ids=[c[0] for c in FUSED])
def test_fwd_router_fused(name, T, H, F, E, k, el, e0, mode):
    """moe_fwd_router: the routing is exactly the oracle's routing of the logits the call returns, those
    logits are the router projection within 1e-5, and y is bitwise moe_fwd's on those logits."""
    print(f"case fwd_router {name} T={T} H={H} E={E} k={k} mode={mode}", flush=True)
    cfg, L = inputs.custom_layer(T=T, H=H, F=F, E=E, k=k, E_local=-1 if el is None else el, e0=e0, seed=61)
    wr = inputs.router_weight(cfg)
    dt = torch.bfloat16
    x, wrd = to_dev(L["x"], dt), to_dev(wr, dt)
    wg, wu, wd = to_dev(L["wg"], dt), to_dev(L["wu"], dt), to_dev(L["wd"], dt)
    layer = MoELayer(T, H, F, E, k, mode, cfg.el, cfg.e0)
    y, lg = layer.forward_router(x, wrd, wg, wu, wd)
    torch.cuda.synchronize()
    lg_np = lg.cpu().numpy()
    rt = {n: t.numpy() for n, t in layer.routing().items()}
    r = oracle.route(lg_np, k, cfg.e0, cfg.el)
    for n in ("idx", "counts", "offsets", "perm", "pair_pos"):
        assert np.array_equal(rt[n], r[n]), n
    assert np.max(np.abs(rt["weight"] - r["w"])) <= 1e-6
    assert oracle.rel_frobenius(lg_np, oracle.router_forward(L["x"], wr)) <= TOL_LOGITS
    ref = MoELayer(T, H, F, E, k, mode, cfg.el, cfg.e0)
    y2 = ref.forward(x, lg, wg, wu, wd)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16)), "y differs from moe_fwd on the same logits"
    # moe_router_fwd runs the same projection: moe_router_fwd + moe_fwd routes exactly as moe_fwd_router
    lg2 = ref.router_forward(x, wrd)
    torch.cuda.synchronize()
    assert torch.equal(lg2, lg), "moe_router_fwd's logits differ from moe_fwd_router's"


@pytest.mark.slow
@pytest.mark.timeout(300)
def test_fwd_router_fused_benchmark_shape():
    cfg = inputs.CONFIGS["qwen3_30b_a3b"]
    print("case fwd_router qwen3_30b_a3b", flush=True)
    x_np, _, _ = inputs.make_tokens(cfg)
    wr = inputs.router_weight(cfg)
    x, wrd = to_dev(x_np, torch.bfloat16), to_dev(wr, torch.bfloat16)
    layer = MoELayer(cfg.T, cfg.H, cfg.F, cfg.E, cfg.k, "bf16")
    lg = torch.empty(cfg.T, cfg.E, dtype=torch.float32, device="cuda")
    # the routing alone (the expert weights do not matter for it): zero weights keep the call cheap
    z = torch.zeros(cfg.E, cfg.F, cfg.H, dtype=torch.bfloat16, device="cuda")
    zd = torch.zeros(cfg.E, cfg.H, cfg.F, dtype=torch.bfloat16, device="cuda")
    layer.forward_router(x, wrd, z, z, zd, logits=lg)
    torch.cuda.synchronize()
    lg_np = lg.cpu().numpy()
    rt = {n: t.numpy() for n, t in layer.routing().items()}
    r = oracle.route(lg_np, cfg.k)
    for n in ("idx", "counts", "offsets", "perm", "pair_pos"):
        assert np.array_equal(rt[n], r[n]), n
    assert oracle.rel_frobenius(lg_np, oracle.router_forward(x_np, wr)) <= TOL_LOGITS


@pytest.mark.parametrize("mode", ["bf16", "mxfp8"])
def test_fwd_router_then_recomputing_backward(mode):
    """moe_fwd_router under activation checkpointing (recompute = 1), then moe_bwd: every gradient is
    bitwise the one of the stored-activation layer run on the same logits, and the layer matches the
    oracle on the logits the fused call returned."""
    T, H, F, E, k = 333, 512, 256, 64, 4
    print(f"case fwd_router + recompute mode={mode}", flush=True)
    cfg, L = inputs.custom_layer(T=T, H=H, F=F, E=E, k=k, seed=71)
    wr = inputs.router_weight(cfg)
    dt = torch.bfloat16
    x, wrd, dy = to_dev(L["x"], dt), to_dev(wr, dt), to_dev(L["dy"], dt)
    wg, wu, wd = to_dev(L["wg"], dt), to_dev(L["wu"], dt), to_dev(L["wd"], dt)
    ck = MoELayer(T, H, F, E, k, mode, recompute=True)
    y, lg = ck.forward_router(x, wrd, wg, wu, wd)
    g = ck.backward(dy, x, wg, wu, wd)
    ref = MoELayer(T, H, F, E, k, mode)
    y2 = ref.forward(x, lg, wg, wu, wd)
    g2 = ref.backward(dy, x, wg, wu, wd)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))
    for n in ("dx", "dw_gate", "dw_up", "dw_down"):
        assert torch.equal(g[n].view(torch.int16), g2[n].view(torch.int16)), n
    assert torch.equal(g["dlogits"], g2["dlogits"])
    lg_np = lg.cpu().numpy()
    args = dict(x=L["x"], logits=lg_np, wg=L["wg"], wu=L["wu"], wd=L["wd"], k=k,
                mode=None if mode == "bf16" else mode)
    ry, _ = oracle.forward(**args)
    rg, _ = oracle.backward(dy=L["dy"], **args)
    tol = 1e-2 if mode == "bf16" else 5e-2
    for n, got, want in (("y", y, ry), ("dx", g["dx"], rg["dx"]), ("dlogits", g["dlogits"], rg["dlogits"]),
                         ("dw_gate", g["dw_gate"], rg["dwg"]), ("dw_up", g["dw_up"], rg["dwu"]),
                         ("dw_down", g["dw_down"], rg["dwd"])):
        err = oracle.rel_frobenius(got.float().cpu().numpy(), want)
        assert err <= tol, (n, err)
