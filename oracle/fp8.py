"""Number formats used by the layer: OCP FP8 e4m3fn and bfloat16.  Test infrastructure only.

e4m3fn (OCP 8-bit floating point specification, E4M3 variant): 1 sign bit, 4 exponent
bits with bias 7, 3 mantissa bits.  Normal values (exponent field e in 1..15):
(-1)^s * 2^(e-7) * (1 + m/8); subnormals (e = 0): (-1)^s * 2^-6 * (m/8).  The codes with
e = 15 and m = 7 (0x7F, 0xFF) are NaN; there is no infinity; the largest finite value is
448 (0x7E).  The pages quantise tokens, intermediate activations and weights to "FP8 e4m3"
with fp32 block scales ("Mega-MoE notes, part 2", 5.2; "Mega-MoE kernel code
walkthrough", section 6).
"""
import numpy as np

E4M3_MAX = 448.0


def e4m3fn_decode(codes) -> np.ndarray:
    """uint8 codes -> float64 values (NaN for 0x7F / 0xFF)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c >> 7, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    normal = np.ldexp(1.0 + m / 8.0, (e - 7).astype(np.int64))
    subnormal = np.ldexp(m / 8.0, -6)
    val = sign * np.where(e == 0, subnormal, normal)
    return np.where((e == 15) & ((c & 7) == 7), np.nan, val)


def e4m3fn_encode(v) -> np.ndarray:
    """float values -> uint8 e4m3fn codes, round to nearest even, saturating to +-448.

    The input is taken exactly as given (callers pass fp32 values when the decision must be
    taken in fp32).  NaN maps to 0x7F.
    """
    x = np.asarray(v, dtype=np.float64)
    sign = np.signbit(x)
    a = np.minimum(np.abs(np.nan_to_num(x, nan=0.0)), E4M3_MAX)            # saturate to the largest finite value
    _, ex = np.frexp(a)                             # a = f * 2^ex with f in [0.5, 1)
    # Exponent of the leading bit is ex-1; values below 2^-6 share the subnormal quantum.
    lead = np.maximum(ex - 1, -6)
    quantum = np.ldexp(1.0, (lead - 3).astype(np.int64))     # 3 mantissa bits
    n = np.rint(a / quantum)                         # exact division, ties to even
    r = n * quantum                                  # rounded magnitude (<= 448)
    # Re-encode the rounded magnitude: exponent field and mantissa.
    _, ex2 = np.frexp(r)
    lead2 = ex2 - 1
    is_sub = (r < 2.0 ** -6)
    efield = np.where(is_sub, 0, lead2 + 7)
    mfield = np.where(is_sub, np.rint(r / 2.0 ** -9),
                      np.rint((r / np.ldexp(1.0, lead2.astype(np.int64)) - 1.0) * 8.0))
    code = (efield.astype(np.int64) << 3) | mfield.astype(np.int64)
    code = np.where(r == 0, 0, code)
    code = code | (sign.astype(np.int64) << 7)
    code = np.where(np.isnan(x), 0x7F, code)
    return code.astype(np.uint8)


def bf16_round(v) -> np.ndarray:
    """Round values to the nearest bfloat16 (8 significant bits, ties to even); float64 out."""
    x = np.asarray(v, dtype=np.float64)
    _, ex = np.frexp(x)
    lead = np.maximum(ex - 1, -126)
    quantum = np.ldexp(1.0, (lead - 7).astype(np.int64))     # 7 stored mantissa bits
    out = np.rint(x / quantum) * quantum
    return np.where(np.isfinite(x), out, x)


def bf16_bits(v) -> np.ndarray:
    """bfloat16 bit patterns (uint16) of values that are already bf16-representable."""
    f32 = np.asarray(v, dtype=np.float64).astype(np.float32)
    return (f32.view(np.uint32) >> 16).astype(np.uint16)
