"""GPU: the layer's forward+backward captured in a HIP graph (torch.cuda.CUDAGraph) and replayed.

The library enqueues kernels only (no allocation, memset, copy or host synchronisation inside
moe_fwd / moe_bwd / moe_route_static), so a caller may capture a whole step. Each replay is checked
bitwise against the eager step on the same inputs, with eager work on the outputs between replays
(they are cleared by torch fill kernels outside the graph), and the eager step is re-run between
replays too. The routing without a workspace (moe_route_static) is captured the same way.
"""
import numpy as np
import pytest
import torch

from mixture_experts_layer_32_amd import binding, inputs
from mixture_experts_layer_32_amd.layer import MoELayer

pytestmark = pytest.mark.gpu

OUTS = ("y", "dx", "dlogits", "dw_gate", "dw_up", "dw_down")


def _snapshot(t):
    return {n: v.view(torch.uint8).clone() for n, v in t.items()}


@pytest.mark.parametrize("mode,recompute,share", [
    ("bf16", False, False), ("mxfp8", False, False), ("fp32", False, False),
    ("bf16", True, False), ("mxfp8", True, False), ("fp32", True, False),
    ("fp8", False, False), ("fp8_bwd", False, False), ("bf16", False, True), ("mxfp8", True, True)])
def test_step_replays_bitwise(mode, recompute, share):
    print(f"case graph step mode={mode} recompute={recompute} share={share}", flush=True)
    cfg, L = inputs.custom_layer(T=333, H=512, F=256, E=16, k=4, dtype="fp32" if mode == "fp32" else "bf16",
                                 seed=81, E_local=4 if share else -1, e0=8 if share else 0)
    dt = torch.float32 if mode == "fp32" else torch.bfloat16
    dev = lambda a, t=dt: torch.from_numpy(np.ascontiguousarray(a)).to("cuda").to(t)
    x, dy, lg = dev(L["x"]), dev(L["dy"]), dev(L["logits"], torch.float32)
    wg, wu, wd = dev(L["wg"]), dev(L["wu"]), dev(L["wd"])
    layer = MoELayer(cfg.T, cfg.H, cfg.F, cfg.E, cfg.k, mode, cfg.el, cfg.e0, recompute=recompute)
    out = dict(y=torch.empty(cfg.T, cfg.H, dtype=dt, device="cuda"), dx=torch.empty_like(x),
               dlogits=torch.empty(cfg.T, cfg.E, dtype=torch.float32, device="cuda"),
               dw_gate=torch.empty_like(wg), dw_up=torch.empty_like(wu), dw_down=torch.empty_like(wd))

    def step():
        layer.forward(x, lg, wg, wu, wd, out["y"])
        layer.backward(dy, x, wg, wu, wd, out={n: out[n] for n in OUTS[1:]})

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    ref = _snapshot(out)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for r in range(3):
        for v in out.values():
            v.zero_()
        graph.replay()
        torch.cuda.synchronize()
        got = _snapshot(out)
        for n in OUTS:
            assert torch.equal(got[n], ref[n]), (r, n)
        step()                      # eager work between the replays
        torch.cuda.synchronize()
        got = _snapshot(out)
        for n in OUTS:
            assert torch.equal(got[n], ref[n]), ("eager", r, n)


def test_route_static_replays_bitwise():
    print("case graph moe_route_static", flush=True)
    T, E, k = 1000, 64, 6
    rng = np.random.default_rng(82)
    lg = torch.from_numpy(rng.standard_normal((T, E)).astype(np.float32)).to("cuda")
    d = binding.Desc.make(T, 256, 128, E, k, "bf16")
    _, _, saved = binding.query_sizes(d)
    sa = torch.full((saved,), 0xFF, dtype=torch.uint8, device="cuda")   # regions it leaves alone stay so
    binding.moe_route_static(d, lg, sa)
    torch.cuda.synchronize()
    ref = sa.clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        binding.moe_route_static(d, lg, sa)
    torch.cuda.synchronize()
    for r in range(3):
        sa.fill_(0xFF)
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(sa, ref), r
