"""ctypes binding of libmoe.so (include/moe.h). Argument marshalling only.

Every step of the layer runs in the HIP library. The functions here take torch tensors (or raw
integer addresses) and hand their device pointers to the C entry points of the same names. If
the library is missing, loading it raises: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
import re

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmoe.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "moe.h")

MODES = {"fp32": 0, "bf16": 1, "mxfp8": 2, "fp8_bwd": 3, "fp8": 4}
STATUS = {0: "MOE_OK", 1: "MOE_ERR_INVALID_ARG", 2: "MOE_ERR_UNSUPPORTED_SHAPE",
          3: "MOE_ERR_UNSUPPORTED_MODE", 4: "MOE_ERR_WORKSPACE_TOO_SMALL", 5: "MOE_ERR_HIP"}


class Desc(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("H", ctypes.c_int32), ("F", ctypes.c_int32),
                ("E_total", ctypes.c_int32), ("E_local", ctypes.c_int32),
                ("expert_offset", ctypes.c_int32), ("topk", ctypes.c_int32), ("mode", ctypes.c_int32),
                ("recompute", ctypes.c_int32)]

    @classmethod
    def make(cls, T, H, F, E_total, topk, mode="bf16", E_local=None, expert_offset=0, recompute=False):
        m = MODES[mode] if isinstance(mode, str) else int(mode)
        return cls(T, H, F, E_total, E_total - expert_offset if E_local is None else E_local,
                   expert_offset, topk, m, int(recompute))


class SavedOffsets(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in ("idx", "weight", "counts", "offsets", "perm", "pair_pos", "qoff", "qcols",
                                               "hwt", "hwt_scales", "wdt", "wdt_scales", "wgut", "wgut_scales")]


class MoEError(RuntimeError):
    def __init__(self, status, detail):
        self.status = status
        self.code = STATUS.get(status, str(status))
        super().__init__(f"{self.code}: {detail}")


_lib = None
_P = ctypes.c_void_p
_D = ctypes.POINTER(Desc)


def header_functions():
    """Names of the functions declared in include/moe.h."""
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\**\s*(moe_\w+)\s*\(", text, re.M)))


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m mixture_experts_layer_32_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        st = ctypes.c_int
        L.moe_query_sizes.argtypes = [_D, ctypes.POINTER(ctypes.c_size_t), ctypes.POINTER(ctypes.c_size_t),
                                      ctypes.POINTER(ctypes.c_size_t)]
        L.moe_route.argtypes = [_D, _P, _P, _P, ctypes.c_size_t, _P]
        L.moe_route_static.argtypes = [_D, _P, _P, _P]
        L.moe_fwd.argtypes = [_D, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]
        L.moe_fwd_router.argtypes = [_D, _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]
        L.moe_bwd.argtypes = [_D, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]
        L.moe_saved_layout.argtypes = [_D, ctypes.POINTER(SavedOffsets)]
        L.moe_status_string.argtypes = [st]
        L.moe_status_string.restype = ctypes.c_char_p
        L.moe_last_error.argtypes = []
        L.moe_last_error.restype = ctypes.c_char_p
        L.moe_version.restype = ctypes.c_char_p
        L.moe_mx_quantize.argtypes = [_P, ctypes.c_int64, ctypes.c_int64, ctypes.c_int, _P, _P, _P]
        L.moe_fp8_block_quantize.argtypes = [_P, ctypes.c_int64, ctypes.c_int64, ctypes.c_int, _P, _P, _P, _P, _P]
        L.moe_query_router_sizes.argtypes = [_D, ctypes.POINTER(ctypes.c_size_t), ctypes.POINTER(ctypes.c_size_t)]
        L.moe_router_fwd.argtypes = [_D, _P, _P, _P, _P, ctypes.c_size_t, _P]
        L.moe_router_bwd.argtypes = [_D, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]
        L.moe_profile_enable.argtypes = [ctypes.c_int]
        L.moe_profile_kernel.argtypes = [ctypes.c_int, ctypes.POINTER(ctypes.c_char_p),
                                         ctypes.POINTER(ctypes.c_int), ctypes.POINTER(ctypes.c_double)]
        for n in ("moe_query_sizes", "moe_route", "moe_route_static", "moe_fwd", "moe_fwd_router", "moe_bwd", "moe_saved_layout", "moe_mx_quantize",
                  "moe_fp8_block_quantize",
                  "moe_query_router_sizes", "moe_router_fwd", "moe_router_bwd", "moe_profile_enable",
                  "moe_profile_disable", "moe_profile_collect", "moe_profile_kernel"):
            getattr(L, n).restype = st
        _lib = L
    return _lib


def _check(status):
    if status != 0:
        raise MoEError(status, lib().moe_last_error().decode())


def ptr(t):
    """Device (or host) address of a tensor, an int address, or None (NULL)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def version():
    return lib().moe_version().decode()


def query_sizes(desc: Desc):
    f, b, s = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    _check(lib().moe_query_sizes(ctypes.byref(desc), ctypes.byref(f), ctypes.byref(b), ctypes.byref(s)))
    return f.value, b.value, s.value


def saved_layout(desc: Desc) -> dict:
    o = SavedOffsets()
    _check(lib().moe_saved_layout(ctypes.byref(desc), ctypes.byref(o)))
    return {n: getattr(o, n) for n, _ in SavedOffsets._fields_}


def moe_route(desc, logits, saved, ws, ws_bytes, stream=None):
    _check(lib().moe_route(ctypes.byref(desc), ptr(logits), ptr(saved), ptr(ws), ws_bytes, _stream(stream)))


def moe_route_static(desc, logits, saved, stream=None):
    _check(lib().moe_route_static(ctypes.byref(desc), ptr(logits), ptr(saved), _stream(stream)))


def moe_fwd(desc, x, logits, w_gate, w_up, w_down, y, saved, ws, ws_bytes, stream=None):
    _check(lib().moe_fwd(ctypes.byref(desc), ptr(x), ptr(logits), ptr(w_gate), ptr(w_up), ptr(w_down), ptr(y),
                         ptr(saved), ptr(ws), ws_bytes, _stream(stream)))


def moe_fwd_router(desc, x, w_router, logits, w_gate, w_up, w_down, y, saved, ws, ws_bytes, stream=None):
    _check(lib().moe_fwd_router(ctypes.byref(desc), ptr(x), ptr(w_router), ptr(logits), ptr(w_gate), ptr(w_up),
                                ptr(w_down), ptr(y), ptr(saved), ptr(ws), ws_bytes, _stream(stream)))


def moe_bwd(desc, dy, x, w_gate, w_up, w_down, saved, dx, dlogits, dw_gate, dw_up, dw_down, ws, ws_bytes,
            stream=None):
    _check(lib().moe_bwd(ctypes.byref(desc), ptr(dy), ptr(x), ptr(w_gate), ptr(w_up), ptr(w_down), ptr(saved),
                         ptr(dx), ptr(dlogits), ptr(dw_gate), ptr(dw_up), ptr(dw_down), ptr(ws), ws_bytes,
                         _stream(stream)))


def query_router_sizes(desc: Desc):
    f, b = ctypes.c_size_t(), ctypes.c_size_t()
    _check(lib().moe_query_router_sizes(ctypes.byref(desc), ctypes.byref(f), ctypes.byref(b)))
    return f.value, b.value


def moe_router_fwd(desc, x, w_router, logits, ws, ws_bytes, stream=None):
    _check(lib().moe_router_fwd(ctypes.byref(desc), ptr(x), ptr(w_router), ptr(logits), ptr(ws), ws_bytes,
                                _stream(stream)))


def moe_router_bwd(desc, x, w_router, dlogits, dx, dw_router, ws, ws_bytes, stream=None):
    _check(lib().moe_router_bwd(ctypes.byref(desc), ptr(x), ptr(w_router), ptr(dlogits), ptr(dx), ptr(dw_router),
                                ptr(ws), ws_bytes, _stream(stream)))


def moe_mx_quantize(x, rows, cols, axis, q, scales, stream=None):
    _check(lib().moe_mx_quantize(ptr(x), rows, cols, axis, ptr(q), ptr(scales), _stream(stream)))


def moe_fp8_block_quantize(x, rows, cols, weight, q, scales, qt=None, scales_t=None, stream=None):
    _check(lib().moe_fp8_block_quantize(ptr(x), rows, cols, int(weight), ptr(q), ptr(scales), ptr(qt), ptr(scales_t),
                                        _stream(stream)))


def profile_enable(max_launches=4096):
    _check(lib().moe_profile_enable(max_launches))


def profile_disable():
    _check(lib().moe_profile_disable())


def profile_collect() -> dict:
    """{kernel name: (launches, total ms)} of the launches recorded since profile_enable()."""
    L = lib()
    _check(L.moe_profile_collect())
    out = {}
    i = 0
    while True:
        name, n, ms = ctypes.c_char_p(), ctypes.c_int(), ctypes.c_double()
        if L.moe_profile_kernel(i, ctypes.byref(name), ctypes.byref(n), ctypes.byref(ms)) != 0:
            break
        out[name.value.decode()] = (n.value, ms.value)
        i += 1
    return out
