"""MXFP4 weight decoding for the FP8 x FP4 variant of the layer.  Test infrastructure only.

The pages name an FP8 x FP4 Mega-MoE kernel and pass its weight scale factors packed along K
("DeepGEMM Mega MoE symmetric memory deep analysis", 10.1-10.2: the FP8/FP4 entry point and the
packed SF layout it transposes).  They do not spell out the element format or the scale block.  The
reading taken here is the plain one for FP4 weights with packed per-K scale factors, OCP MXFP4:
  * elements are e2m1: 1 sign bit, 2 exponent bits with bias 1, 1 mantissa bit, no infinities or
    NaN.  Magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6 (exponent 0 is subnormal: 0.5 * mantissa);
  * one UE8M0 scale per 32 consecutive values along K: an unsigned 8-bit exponent, value 2^(e - 127),
    with 255 = NaN;
  * W[n, k] = e2m1(code[n, k]) * 2^(scale[n, k / 32] - 127).
Two e2m1 codes share a byte, the element with the lower K index in the low nibble.
"""
from __future__ import annotations

import numpy as np

E2M1_MAX = 6.0
MX_BLOCK = 32


def e2m1_decode(codes) -> np.ndarray:
    """4-bit e2m1 codes (0..15, higher bits ignored) -> float64."""
    c = np.asarray(codes).astype(np.uint8) & 0xF
    sign = np.where(c & 0x8, -1.0, 1.0)
    e = ((c >> 1) & 0x3).astype(np.int64)
    m = (c & 0x1).astype(np.float64)
    mag = np.where(e == 0, 0.5 * m, np.ldexp(1.0 + 0.5 * m, (e - 1).astype(np.int64)))
    return sign * mag


def e8m0_decode(scales) -> np.ndarray:
    """UE8M0 scale bytes -> float64 2^(e - 127); 255 is NaN."""
    e = np.asarray(scales).astype(np.int64)
    v = np.ldexp(1.0, e - 127)
    return np.where(e == 255, np.nan, v)


def unpack_fp4(packed: np.ndarray, k: int) -> np.ndarray:
    """[..., k/2] bytes -> [..., k] codes, the lower K index in the low nibble."""
    p = np.asarray(packed).astype(np.uint8)
    out = np.empty(p.shape[:-1] + (k,), dtype=np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out


def dequant_mx(packed: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """MXFP4 weight [N, K/2] packed codes + [N, K/32] UE8M0 scales -> float64 [N, K]."""
    k = packed.shape[-1] * 2
    codes = unpack_fp4(packed, k)
    s = np.repeat(e8m0_decode(scales), MX_BLOCK, axis=-1)
    return e2m1_decode(codes) * s
