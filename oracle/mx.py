"""MXFP8 emulation for the float64 oracle. TEST INFRASTRUCTURE ONLY (same rules as moe_oracle).

The pages name MXFP8 as one of the kernel's precision modes ("Supporto di precisione e vincoli
hardware" on "Prime Mega MoE: il kernel che accelera il training AI del 55%"; "A Magia da Fusão" on
"IA: MoE Kernel 3x Mais Rápido Chegou!"). They give no details. The format read here is the OCP
microscaling one:
 * blocks of 32 consecutive elements along a GEMM's contraction axis share one power-of-two scale
   X = 2^s, stored as e8m0 (s in [-127, 127]);
 * elements are FP8 E4M3 in its finite-only form: bias 7, largest value 448, smallest subnormal
   2^-9, no infinities.
 * s = floor(log2(amax)) - 8, where 8 is the exponent of E4M3's largest normal. A block whose
   amax is zero gets s = -127 and zero elements.
 * elements = E4M3(v / X), rounded to nearest with ties to even, and saturated to +-448.

Quantisation only replaces GEMM operands (quantise, then dequantise in float64). Every other step
stays exact.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
E4M3_EMAX = 8          # exponent of the largest normal E4M3 value (1.75 * 2^8)
E4M3_EMIN = -6         # exponent of the smallest normal
E4M3_MBITS = 3
BLOCK = 32


def e4m3_round(v):
    """Nearest E4M3 value (ties to even), saturated to +-448. float64 in, float64 out."""
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    _, ex = np.frexp(a)                       # a = m * 2^ex with m in [0.5, 1)
    e = np.maximum(ex - 1, E4M3_EMIN)         # floor(log2 a), held at the subnormal exponent
    step = np.ldexp(1.0, e - E4M3_MBITS)      # spacing of E4M3 values in that binade
    q = np.round(a / step) * step             # numpy rounds halves to even
    q = np.minimum(q, E4M3_MAX)
    return np.where(a == 0, 0.0, np.copysign(q, v))


def block_scale_exponent(amax):
    """e8m0 exponent s per block: floor(log2 amax) - 8, clamped to [-127, 127]; -127 if amax == 0."""
    amax = np.asarray(amax, dtype=np.float64)
    _, ex = np.frexp(amax)
    s = np.clip(ex - 1 - E4M3_EMAX, -127, 127)
    return np.where(amax == 0, -127, s).astype(np.int64)


def mx_quantize(v, axis=-1, return_parts=False):
    """MXFP8 round trip of v along `axis` in blocks of 32.

    A last block shorter than 32 is padded with zeros. Returns the dequantised float64 array,
    plus (elements, scale exponents) if return_parts.
    """
    v = np.asarray(v, dtype=np.float64)
    x = np.moveaxis(v, axis, -1)
    n = x.shape[-1]
    nb = -(-n // BLOCK)
    pad = nb * BLOCK - n
    if pad:
        x = np.concatenate([x, np.zeros(x.shape[:-1] + (pad,))], axis=-1)
    blocks = x.reshape(x.shape[:-1] + (nb, BLOCK))
    s = block_scale_exponent(np.max(np.abs(blocks), axis=-1))
    scale = np.ldexp(1.0, s)[..., None]
    elems = e4m3_round(blocks / scale)
    deq = (elems * scale).reshape(x.shape)[..., :n]
    out = np.moveaxis(deq, -1, axis)
    if return_parts:
        return out, np.moveaxis(elems.reshape(x.shape)[..., :n], -1, axis), s
    return out


def e4m3_table():
    """The 254 finite values of E4M3 (finite-only form), decoded from their bit fields."""
    vals = []
    for code in range(256):
        sign = -1.0 if code & 0x80 else 1.0
        exp = (code >> 3) & 0xF
        man = code & 0x7
        if exp == 0xF and man == 0x7:
            continue                           # the NaN encodings
        if exp == 0:
            vals.append(sign * man / 8.0 * 2.0 ** (1 - 7))
        else:
            vals.append(sign * (1.0 + man / 8.0) * 2.0 ** (exp - 7))
    return np.array(vals)
