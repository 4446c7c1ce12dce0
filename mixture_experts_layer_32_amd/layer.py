"""Device-memory plumbing around the C ABI: torch allocates the caller-owned buffers.

MoELayer holds the workspace and saved buffers for one layer shape, and calls moe_fwd/moe_bwd (and
the router projection's moe_router_fwd/moe_router_bwd) through the binding. No arithmetic happens
here.
"""
from __future__ import annotations

import torch

from . import binding


def _expect(t, name, shape, dtype, device):
    """Raises ValueError unless t is a contiguous tensor of this shape and dtype on this device: the
    C ABI receives bare pointers and cannot check any of it."""
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name}: expected a torch.Tensor, got {type(t).__name__}")
    if t.device != device:
        raise ValueError(f"{name}: expected a tensor on {device}, got {t.device}")
    if t.dtype != dtype:
        raise ValueError(f"{name}: expected dtype {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: expected a contiguous tensor")


class MoELayer:
    def __init__(self, T, H, F, E_total, topk, mode="bf16", E_local=None, expert_offset=0, device="cuda",
                 recompute=False):
        """recompute=True: activation checkpointing (the backward recomputes the gate/up activations
        from x instead of reading them from the saved buffer)."""
        self.desc = binding.Desc.make(T, H, F, E_total, topk, mode, E_local, expert_offset, recompute)
        self.mode = mode
        self.dtype = torch.float32 if mode == "fp32" else torch.bfloat16
        self.device = torch.device(device)
        if self.device.type == "cuda" and self.device.index is None:
            self.device = torch.device("cuda", torch.cuda.current_device())
        self.fwd_ws_bytes, self.bwd_ws_bytes, self.saved_bytes = binding.query_sizes(self.desc)
        u8 = dict(dtype=torch.uint8, device=self.device)
        self.ws = torch.empty(max(self.fwd_ws_bytes, self.bwd_ws_bytes), **u8)
        self.saved = torch.empty(self.saved_bytes, **u8)

    @property
    def shape(self):
        d = self.desc
        return dict(T=d.T, H=d.H, F=d.F, E=d.E_total, E_local=d.E_local, e0=d.expert_offset, k=d.topk)

    def _check(self, **tensors):
        d, el, f32 = self.desc, self.dtype, torch.float32
        spec = dict(x=((d.T, d.H), el), y=((d.T, d.H), el), dy=((d.T, d.H), el), dx=((d.T, d.H), el),
                    logits=((d.T, d.E_total), f32), dlogits=((d.T, d.E_total), f32),
                    w_gate=((d.E_local, d.F, d.H), el), w_up=((d.E_local, d.F, d.H), el),
                    w_down=((d.E_local, d.H, d.F), el), dw_gate=((d.E_local, d.F, d.H), el),
                    dw_up=((d.E_local, d.F, d.H), el), dw_down=((d.E_local, d.H, d.F), el),
                    w_router=((d.E_total, d.H), el), dw_router=((d.E_total, d.H), el))
        for name, t in tensors.items():
            shape, dtype = spec[name]
            _expect(t, name, shape, dtype, self.device)

    def forward(self, x, logits, w_gate, w_up, w_down, y=None, stream=None):
        d = self.desc
        if y is None:
            y = torch.empty(d.T, d.H, dtype=self.dtype, device=self.device)
        self._check(x=x, logits=logits, w_gate=w_gate, w_up=w_up, w_down=w_down, y=y)
        binding.moe_fwd(d, x, logits, w_gate, w_up, w_down, y, self.saved, self.ws, self.ws.numel(), stream)
        return y

    def forward_router(self, x, w_router, w_gate, w_up, w_down, y=None, logits=None, stream=None):
        """The forward from x through moe_fwd_router (router projection fused with the routing);
        returns (y, logits)."""
        d = self.desc
        if y is None:
            y = torch.empty(d.T, d.H, dtype=self.dtype, device=self.device)
        if logits is None:
            logits = torch.empty(d.T, d.E_total, dtype=torch.float32, device=self.device)
        self._check(x=x, w_router=w_router, logits=logits, w_gate=w_gate, w_up=w_up, w_down=w_down, y=y)
        binding.moe_fwd_router(d, x, w_router, logits, w_gate, w_up, w_down, y, self.saved, self.ws, self.ws.numel(),
                               stream)
        return y, logits

    def route(self, logits, stream=None):
        self._check(logits=logits)
        binding.moe_route(self.desc, logits, self.saved, self.ws, self.ws.numel(), stream)

    def backward(self, dy, x, w_gate, w_up, w_down, out=None, stream=None):
        d = self.desc
        if out is None:
            kw = dict(dtype=self.dtype, device=self.device)
            out = dict(dx=torch.empty(d.T, d.H, **kw),
                       dlogits=torch.empty(d.T, d.E_total, dtype=torch.float32, device=self.device),
                       dw_gate=torch.empty(d.E_local, d.F, d.H, **kw),
                       dw_up=torch.empty(d.E_local, d.F, d.H, **kw),
                       dw_down=torch.empty(d.E_local, d.H, d.F, **kw))
        self._check(dy=dy, x=x, w_gate=w_gate, w_up=w_up, w_down=w_down, dx=out["dx"], dlogits=out["dlogits"],
                    dw_gate=out["dw_gate"], dw_up=out["dw_up"], dw_down=out["dw_down"])
        binding.moe_bwd(d, dy, x, w_gate, w_up, w_down, self.saved, out["dx"], out["dlogits"], out["dw_gate"],
                        out["dw_up"], out["dw_down"], self.ws, self.ws.numel(), stream)
        return out

    def _router_ws(self):
        if getattr(self, "router_ws", None) is None:
            f, b = binding.query_router_sizes(self.desc)
            self.router_ws = torch.empty(max(f, b, 256), dtype=torch.uint8, device=self.device)
        return self.router_ws

    def router_forward(self, x, w_router, logits=None, stream=None):
        """logits = x w_router^T (fp32) through moe_router_fwd; w_router [E_total, H]."""
        d = self.desc
        if logits is None:
            logits = torch.empty(d.T, d.E_total, dtype=torch.float32, device=self.device)
        self._check(x=x, w_router=w_router, logits=logits)
        ws = self._router_ws()
        binding.moe_router_fwd(d, x, w_router, logits, ws, ws.numel(), stream)
        return logits

    def router_backward(self, x, w_router, dlogits, dx, dw_router=None, stream=None):
        """dw_router = dlogits^T x (returned), and dx += dlogits w_router in place."""
        d = self.desc
        if dw_router is None:
            dw_router = torch.empty(d.E_total, d.H, dtype=self.dtype, device=self.device)
        self._check(x=x, w_router=w_router, dlogits=dlogits, dx=dx, dw_router=dw_router)
        ws = self._router_ws()
        binding.moe_router_bwd(d, x, w_router, dlogits, dx, dw_router, ws, ws.numel(), stream)
        return dw_router

    def routing(self):
        """Routing results from `saved` as CPU tensors: idx, weight, counts, offsets, perm, pair_pos."""
        d = self.desc
        off = binding.saved_layout(d)
        rows = d.T * d.topk
        s = self.saved

        def view(name, n, dt):
            b = 4 * n
            return s[off[name]:off[name] + b].view(dt).cpu()
        offsets = view("offsets", d.E_local + 1, torch.int32)
        P = int(offsets[-1])
        return dict(idx=view("idx", rows, torch.int32).view(d.T, d.topk),
                    weight=view("weight", rows, torch.float32).view(d.T, d.topk),
                    counts=view("counts", d.E_local, torch.int32), offsets=offsets,
                    perm=view("perm", rows, torch.int32)[:P], pair_pos=view("pair_pos", rows, torch.int32))
