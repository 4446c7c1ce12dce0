"""Pins of the oracle's router projection (logits = x W_r^T in front of the layer; CPU only).

The projection's forward and backward are checked through the whole composition
x, W_r -> logits -> routed layer -> y:
 * against torch float64 autograd of a dense-masked formulation (torch's own matmul and
   autograd, no oracle code);
 * against central finite differences of <dY, y> in W_r and in x (x reaches y both through the
   experts and through the router).
The planted mistakes at the end show that these pins catch a dropped router term in dx and a
sign slip in dW_r.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import oracle.moe_oracle as om


def router_layer(T=20, H=10, F=6, E=6, k=2, seed=11):
    rng = np.random.default_rng(seed)
    return dict(x=rng.standard_normal((T, H)), wr=rng.standard_normal((E, H)) / math.sqrt(H),
                wg=rng.standard_normal((E, F, H)) / math.sqrt(H), wu=rng.standard_normal((E, F, H)) / math.sqrt(H),
                wd=rng.standard_normal((E, H, F)) / math.sqrt(F), dy=rng.standard_normal((T, H)), k=k)


def oracle_composed(L):
    """y, dx (layer + router), dW_r and the experts' gradients from the oracle's functions."""
    lg = oracle.router_forward(L["x"], L["wr"])
    args = dict(x=L["x"], logits=lg, wg=L["wg"], wu=L["wu"], wd=L["wd"], k=L["k"])
    y, _ = oracle.forward(**args)
    g, _ = oracle.backward(dy=L["dy"], **args)
    dwr, dxr = oracle.router_backward(g["dlogits"], L["x"], L["wr"])
    return dict(y=y, dx=g["dx"] + dxr, dwr=dwr, dwg=g["dwg"], dwu=g["dwu"], dwd=g["dwd"])


def torch_composed(L):
    """Dense-masked MoE behind a linear router, torch float64; selection held constant."""
    t = lambda a: torch.tensor(np.asarray(a, np.float64), requires_grad=True)
    x, wr, wg, wu, wd = t(L["x"]), t(L["wr"]), t(L["wg"]), t(L["wu"]), t(L["wd"])
    lg = x @ wr.T
    idx = torch.topk(lg.detach(), L["k"], dim=1).indices
    w = torch.softmax(torch.gather(lg, 1, idx), dim=1)
    y = torch.zeros_like(x)
    for e in range(wg.shape[0]):
        me = (w * (idx == e)).sum(1, keepdim=True)
        h = torch.nn.functional.silu(x @ wg[e].T) * (x @ wu[e].T)
        y = y + me * (h @ wd[e].T)
    (y * torch.from_numpy(np.asarray(L["dy"], np.float64))).sum().backward()
    return dict(y=y.detach().numpy(), dx=x.grad.numpy(), dwr=wr.grad.numpy(), dwg=wg.grad.numpy(),
                dwu=wu.grad.numpy(), dwd=wd.grad.numpy())


def gap_ok(lg, k, margin):
    s = -np.sort(-np.asarray(lg, np.float64), axis=1)
    return k >= s.shape[1] or bool(np.all(s[:, k - 1] - s[:, k] > margin))


@pytest.mark.parametrize("shape", [dict(T=20, H=10, F=6, E=6, k=2), dict(T=13, H=8, F=4, E=8, k=8),
                                   dict(T=17, H=6, F=5, E=3, k=1)])
def test_router_composition_against_torch_autograd(shape):
    L = router_layer(**shape)
    o, tt = oracle_composed(L), torch_composed(L)
    for name in o:
        assert o[name].shape == tt[name].shape, name
        np.testing.assert_allclose(o[name], tt[name], rtol=1e-11, atol=1e-12, err_msg=name)


def fd_router_errors(L, eps=1e-6, seed=3):
    """Relative error of <grad, v> against central differences of <dY, y>, for v along W_r and x."""
    rng = np.random.default_rng(seed)
    g = oracle_composed(L)

    def loss(x, wr):
        y, _ = oracle.forward(x, oracle.router_forward(x, wr), L["wg"], L["wu"], L["wd"], L["k"])
        return np.sum(L["dy"] * y)
    errs = {}
    for name, gname in (("wr", "dwr"), ("x", "dx")):
        v = rng.standard_normal(np.shape(L[name]))
        plus = {"x": L["x"], "wr": L["wr"], name: L[name] + eps * v}
        minus = {"x": L["x"], "wr": L["wr"], name: L[name] - eps * v}
        fd = (loss(**plus) - loss(**minus)) / (2 * eps)
        an = np.sum(g[gname] * v)
        errs[name] = abs(fd - an) / max(abs(an), 1e-30)
    return errs


@pytest.mark.parametrize("shape", [dict(T=16, H=8, F=5, E=6, k=2), dict(T=10, H=6, F=4, E=4, k=3)])
def test_router_finite_differences(shape):
    L = router_layer(**shape)
    # a perturbation of size 1e-6 along a unit-variance direction cannot change the selection
    assert gap_ok(oracle.router_forward(L["x"], L["wr"]), L["k"], 1e-3)
    errs = fd_router_errors(L)
    assert max(errs.values()) < 1e-6, errs


def test_router_projection_shapes_and_linearity():
    L = router_layer(T=7, H=5, E=4)
    lg = oracle.router_forward(L["x"], L["wr"])
    assert lg.shape == (7, 4)
    np.testing.assert_allclose(oracle.router_forward(L["x"], 3.0 * L["wr"]), 3.0 * lg, rtol=1e-14)
    dl = np.random.default_rng(0).standard_normal((7, 4))
    dwr, dxr = oracle.router_backward(dl, L["x"], L["wr"])
    assert dwr.shape == (4, 5) and dxr.shape == (7, 5)
    z = oracle.router_backward(np.zeros((7, 4)), L["x"], L["wr"])
    assert not np.any(z[0]) and not np.any(z[1])


# ------------------------------------------------------------------------------------ the pins bite

def test_planted_mistake_router_dx_term_dropped_is_caught(monkeypatch):
    real = om.router_backward
    monkeypatch.setattr(om, "router_backward", lambda dl, x, wr: (real(dl, x, wr)[0], 0.0 * real(dl, x, wr)[1]))
    monkeypatch.setattr(oracle, "router_backward", om.router_backward)
    errs = fd_router_errors(router_layer(T=16, H=8, F=5, E=6, k=2))
    assert errs["x"] > 1e-3 and errs["wr"] < 1e-6


def test_planted_mistake_router_weight_grad_sign_is_caught(monkeypatch):
    real = om.router_backward
    monkeypatch.setattr(om, "router_backward", lambda dl, x, wr: (-real(dl, x, wr)[0], real(dl, x, wr)[1]))
    monkeypatch.setattr(oracle, "router_backward", om.router_backward)
    errs = fd_router_errors(router_layer(T=16, H=8, F=5, E=6, k=2))
    assert errs["wr"] > 1.0
