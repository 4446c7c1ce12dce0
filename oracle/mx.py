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

Blockwise FP8 (the "fp8" mode). The same pages list a blockwise-scaled FP8 mode for Hopper and give
no block sizes. The reading here is the usual one for FP8 training of this kind of layer, with the
scale restricted to a power of two (an e8m0 byte), which is what the gfx950 scaled MFMA consumes:
 * activation operands: one scale per 128 consecutive elements along the GEMM's contraction axis
   (1 x 128 along a row, or 128 x 1 down an expert's pairs for the weight gradients);
 * weights: one scale per 128 x 128 tile of each expert's matrix, so that both orientations of a
   weight share every scale;
 * the scale is the smallest power of two 2^s with amax <= 448 * 2^s (s clamped to [-127, 127],
   s = -127 for an all-zero block), so no element saturates;
 * elements are E4M3 of v / 2^s, rounded to nearest with ties to even.
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


def ceil_scale_exponent(amax):
    """Blockwise FP8 scale exponent: the smallest s with amax <= 448 * 2^s, clamped to [-127, 127];
    -127 if amax == 0."""
    amax = np.asarray(amax, dtype=np.float64)
    _, ex = np.frexp(amax)
    s = ex - 1 - E4M3_EMAX                          # floor(log2 amax) - 8: amax / 2^s lies in [256, 512)
    s = s + (amax > np.ldexp(E4M3_MAX, s))          # past 448 * 2^s: the next power of two
    s = np.clip(s, -127, 127)
    return np.where(amax == 0, -127, s).astype(np.int64)


def _quantize_blocks(v, axis, block, scale_exponent, return_parts):
    v = np.asarray(v, dtype=np.float64)
    x = np.moveaxis(v, axis, -1)
    n = x.shape[-1]
    nb = -(-n // block)
    pad = nb * block - n
    if pad:
        x = np.concatenate([x, np.zeros(x.shape[:-1] + (pad,))], axis=-1)
    blocks = x.reshape(x.shape[:-1] + (nb, block))
    s = scale_exponent(np.max(np.abs(blocks), axis=-1))
    scale = np.ldexp(1.0, s)[..., None]
    elems = e4m3_round(blocks / scale)
    deq = (elems * scale).reshape(x.shape)[..., :n]
    out = np.moveaxis(deq, -1, axis)
    if return_parts:
        return out, np.moveaxis(elems.reshape(x.shape)[..., :n], -1, axis), s
    return out


def mx_quantize(v, axis=-1, return_parts=False):
    """MXFP8 round trip of v along `axis` in blocks of 32.

    A last block shorter than 32 is padded with zeros. Returns the dequantised float64 array,
    plus (elements, scale exponents) if return_parts.
    """
    return _quantize_blocks(v, axis, BLOCK, block_scale_exponent, return_parts)


FP8_BLOCK = 128


def fp8_block_quantize(v, axis=-1, return_parts=False):
    """Blockwise FP8 round trip of an activation operand along `axis`, in blocks of 128 (the last
    one zero-padded), with the scale rule of ceil_scale_exponent."""
    return _quantize_blocks(v, axis, FP8_BLOCK, ceil_scale_exponent, return_parts)


def fp8_tile_quantize(w, return_parts=False):
    """Blockwise FP8 round trip of a 2-D weight in 128 x 128 tiles, one scale per tile (edge tiles
    are zero-padded). Returns the dequantised array, plus (elements, scale exponents per tile)."""
    w = np.asarray(w, dtype=np.float64)
    R, C = w.shape
    nr, nc = -(-R // FP8_BLOCK), -(-C // FP8_BLOCK)
    pad = np.zeros((nr * FP8_BLOCK, nc * FP8_BLOCK))
    pad[:R, :C] = w
    tiles = pad.reshape(nr, FP8_BLOCK, nc, FP8_BLOCK)
    s = ceil_scale_exponent(np.max(np.abs(tiles), axis=(1, 3)))
    scale = np.ldexp(1.0, s)[:, None, :, None]
    elems = e4m3_round(tiles / scale)
    deq = (elems * scale).reshape(pad.shape)[:R, :C]
    if return_parts:
        return deq, elems.reshape(pad.shape)[:R, :C], s
    return deq


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
