"""Seeded synthetic inputs for the MoE layer: shapes, distributions and encodings only.

Both the HIP path and the float64 reference consume the arrays made here, bit for bit.
This module holds none of the layer's arithmetic (no routing, no expert math): it draws
normal variates, rounds them to the storage precision and, for the router logits, applies
the router projection that sits in front of the layer (logits = x . W_r, plus an optional
per-expert prior).

Workloads (the layer shapes of the Qwen3 MoE models the pages benchmark: 128 experts,
top-8 routing, 16,384-token sequences; "Os Números que Impressionam" on the page
"IA: MoE Kernel 3x Mais Rápido Chegou!" and "Analisi dei kernel layer" on the page
"Prime Mega MoE: il kernel che accelera il training AI del 55%"):

  tiny                 T=256,   H=256,  E=8,   F=128,  k=2, fp32
  qwen3_30b_a3b        T=16384, H=2048, E=128, F=768,  k=8, bf16
  qwen3_30b_a3b_ep16   the same inputs, experts 0..15 only (one rank's expert share)
  qwen3_235b_a22b_zipf T=16384, H=4096, E=128, F=1536, k=8, bf16, Zipf-skewed router prior
  qwen3_30b_a3b_mxfp8  the qwen3_30b_a3b inputs, for the fp8 precision modes (MXFP8, FP8_BWD, FP8)

Distributions: x ~ N(0,1); W_gate, W_up ~ N(0, 1/H); W_down ~ N(0, 1/F) (variance 1/fan_in);
W_r ~ N(0, 0.02^2) (standard deviation 0.02); dY ~ N(0,1). Every tensor is drawn from its
own numpy Generator keyed by (seed, tensor id, expert), so one expert's weights can be
regenerated alone. bf16 workloads round every fp32 draw to bf16 with round-to-nearest-even;
the logits stay fp32.
"""
from __future__ import annotations

import dataclasses
import math
from concurrent.futures import ThreadPoolExecutor

import numpy as np

# tensor ids used as the second word of each Generator key
_TID_X, _TID_WG, _TID_WU, _TID_WD, _TID_WR, _TID_DY = 0, 1, 2, 3, 4, 5


@dataclasses.dataclass(frozen=True)
class LayerConfig:
    name: str
    T: int
    H: int
    F: int
    E: int              # routed experts in total
    k: int              # experts per token
    dtype: str          # "fp32" or "bf16": storage type of x, weights, y and gradients
    seed: int
    E_local: int = -1   # experts computed here (-1: all of them)
    e0: int = 0         # first local expert
    zipf_s: float = 0.0  # >0: add the prior -s*ln(e+1) to expert e's logit

    @property
    def el(self) -> int:
        return self.E if self.E_local < 0 else self.E_local

    def with_(self, **kw) -> "LayerConfig":
        return dataclasses.replace(self, **kw)


CONFIGS = {
    "tiny": LayerConfig("tiny", T=256, H=256, F=128, E=8, k=2, dtype="fp32", seed=0),
    "qwen3_30b_a3b": LayerConfig("qwen3_30b_a3b", T=16384, H=2048, F=768, E=128, k=8,
                                 dtype="bf16", seed=1),
    "qwen3_30b_a3b_ep16": LayerConfig("qwen3_30b_a3b_ep16", T=16384, H=2048, F=768, E=128,
                                      k=8, dtype="bf16", seed=1, E_local=16, e0=0),
    "qwen3_235b_a22b_zipf": LayerConfig("qwen3_235b_a22b_zipf", T=16384, H=4096, F=1536,
                                        E=128, k=8, dtype="bf16", seed=4, zipf_s=1.1),
    "qwen3_30b_a3b_mxfp8": LayerConfig("qwen3_30b_a3b_mxfp8", T=16384, H=2048, F=768, E=128,
                                       k=8, dtype="bf16", seed=1),
}


# ---------------------------------------------------------------------------------------------
# bf16 encoding (storage format, not layer arithmetic)

def round_to_bf16(a: np.ndarray) -> np.ndarray:
    """fp32 -> nearest bf16 (ties to even), returned as fp32 holding a bf16-exact value."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """bf16-exact fp32 array -> its uint16 bf16 encoding (no rounding happens here)."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    if np.any(u & 0xFFFF):
        raise ValueError("array is not bf16-exact")
    return (u >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# ---------------------------------------------------------------------------------------------

def _normal(key, shape, std, bf16):
    v = np.random.default_rng(list(key)).standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        v *= np.float32(std)
    return round_to_bf16(v) if bf16 else v


def expert_weights(cfg: LayerConfig, e: int):
    """(W_gate[e] [F,H], W_up[e] [F,H], W_down[e] [H,F]) of global expert e, fp32 arrays."""
    bf = cfg.dtype == "bf16"
    wg = _normal((cfg.seed, _TID_WG, e), (cfg.F, cfg.H), 1.0 / math.sqrt(cfg.H), bf)
    wu = _normal((cfg.seed, _TID_WU, e), (cfg.F, cfg.H), 1.0 / math.sqrt(cfg.H), bf)
    wd = _normal((cfg.seed, _TID_WD, e), (cfg.H, cfg.F), 1.0 / math.sqrt(cfg.F), bf)
    return wg, wu, wd


def make_weights(cfg: LayerConfig, threads: int = 16):
    """Stacked local-expert weights: W_gate, W_up [E_local,F,H] and W_down [E_local,H,F]."""
    el = cfg.el
    wg = np.empty((el, cfg.F, cfg.H), np.float32)
    wu = np.empty((el, cfg.F, cfg.H), np.float32)
    wd = np.empty((el, cfg.H, cfg.F), np.float32)

    def fill(i):
        wg[i], wu[i], wd[i] = expert_weights(cfg, cfg.e0 + i)

    with ThreadPoolExecutor(max(1, threads)) as ex:
        list(ex.map(fill, range(el)))
    return wg, wu, wd


def _rows(cfg, tid, ncols, std, threads, chunk=1024):
    """[T, ncols] normals drawn in independent 1024-row chunks (keyed by chunk index)."""
    bf = cfg.dtype == "bf16"
    out = np.empty((cfg.T, ncols), np.float32)

    def fill(c):
        r0, r1 = c * chunk, min(cfg.T, (c + 1) * chunk)
        out[r0:r1] = _normal((cfg.seed, tid, c), (r1 - r0, ncols), std, bf)

    with ThreadPoolExecutor(max(1, threads)) as ex:
        list(ex.map(fill, range((cfg.T + chunk - 1) // chunk)))
    return out


def _router_draw(cfg: LayerConfig):
    wr = np.random.default_rng([cfg.seed, _TID_WR, 0]).standard_normal((cfg.H, cfg.E), dtype=np.float32)
    wr *= np.float32(0.02)
    return wr


def router_weight(cfg: LayerConfig):
    """W_r [E, H] (out x in) for the router projection in front of the layer: the draw the logits
    of make_tokens come from, transposed, and rounded to bf16 for bf16 workloads."""
    wr = np.ascontiguousarray(_router_draw(cfg).T)
    return round_to_bf16(wr) if cfg.dtype == "bf16" else wr


def make_tokens(cfg: LayerConfig, threads: int = 16):
    """(x [T,H], logits [T,E] fp32, dy [T,H]); x and dy are bf16-exact for bf16 workloads."""
    x = _rows(cfg, _TID_X, cfg.H, 1.0, threads)
    dy = _rows(cfg, _TID_DY, cfg.H, 1.0, threads)
    wr = _router_draw(cfg)
    # router projection in float64 from the stored x, then fp32 logits
    logits = x.astype(np.float64) @ wr.astype(np.float64)
    if cfg.zipf_s > 0:
        logits += -cfg.zipf_s * np.log(np.arange(1, cfg.E + 1, dtype=np.float64))[None, :]
    return x, logits.astype(np.float32), dy


def make_layer(cfg: LayerConfig, threads: int = 16) -> dict:
    x, logits, dy = make_tokens(cfg, threads)
    wg, wu, wd = make_weights(cfg, threads)
    return dict(x=x, logits=logits, dy=dy, wg=wg, wu=wu, wd=wd)


def custom_layer(T, H, F, E, k, dtype="bf16", seed=123, E_local=-1, e0=0, zipf_s=0.0,
                 threads: int = 8) -> tuple[LayerConfig, dict]:
    """A layer of any shape with the same distributions (used for ragged/edge-case tests)."""
    cfg = LayerConfig(f"custom_T{T}_H{H}_F{F}_E{E}_k{k}", T=T, H=H, F=F, E=E, k=k, dtype=dtype,
                      seed=seed, E_local=E_local, e0=e0, zipf_s=zipf_s)
    return cfg, make_layer(cfg, threads)
