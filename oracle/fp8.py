"""FP8 (E4M3) encoding and static-scale quantization (oracle, test infrastructure).

What is computed.  FlashDecoder review, inference optimisations: static,
calibrated FP8 quantization for matrix products, with a quality cost the
review reports (Table 2, the -Opt rows); the Ultra Flash README mirror's CLI
table offers the same switch (--fp8, --fp8_sr) for its DiT models.  For the
attention path this is read as:
  * q, k and v are quantized to FP8 E4M3 with one static scale per tensor:
    code = E4M3(x * (1 / scale)), the scale a float32, its reciprocal rounded to
    float32 and the product taken in float32, the encoding
    rounding to the nearest representable value (ties to the even code, a
    value that rounds to zero keeping its sign) and saturating at +-448; the
    value is then code * scale.
  * q's scale for attention is the caller's q_scale rounded up, by less than a
    factor of two, so that log2(e)/sqrt(d) * q_scale' * k_scale is a power of two
    (attention_q_scale; the pages fix no rule for it: a static calibration picks
    a scale, and this choice only moves the top of q's range up, never down).
  * The attention itself is the plain definition (oracle.attention.attend)
    applied to those dequantized values in float64.

E4M3 ("FP8 E4M3" of the OCP 8-bit floating point specification): 1 sign bit,
4 exponent bits with bias 7, 3 mantissa bits; exponent field 0 encodes
subnormals m/8 * 2^-6; no infinities; S.1111.111 is NaN, so the largest
finite magnitude is 1.75 * 2^8 = 448.
"""
from __future__ import annotations

import math

import numpy as np

MAX_E4M3 = 448.0


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """uint8 E4M3 codes -> float64 values (NaN for the two NaN codes)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    out = sign * mag
    return np.where((e == 15) & ((c & 7) == 7), np.nan, out)


def e4m3_encode(x: np.ndarray) -> np.ndarray:
    """float32 values -> uint8 E4M3 codes: nearest value, ties to the even code, saturating
    at +-448 (finite inputs only)."""
    x = np.asarray(x, dtype=np.float32).astype(np.float64)
    if not np.isfinite(x).all():
        raise ValueError("e4m3_encode takes finite values")
    sign = np.signbit(x)
    a = np.minimum(np.abs(x), MAX_E4M3)
    # The representable magnitudes below 2^-6 are spaced 2^-9; in [2^e, 2^(e+1)) they are
    # spaced 2^(e-3).  Round |x| / spacing to the nearest integer, ties to even.
    _, fe = np.frexp(a)                      # a = f * 2^fe, f in [0.5, 1): binade e = fe - 1
    e = np.clip(fe - 1, -6, 8).astype(np.float64)
    spacing = np.exp2(e - 3)
    n = np.rint(a / spacing)                 # numpy rounds halves to even; a / spacing is exact
    value = n * spacing                      # n == 16 lands on 2^(e+1), the next binade's first value
    code = np.zeros(a.shape, dtype=np.int64)
    sub = value < 2.0 ** -6
    code[sub] = np.rint(value[sub] / 2.0 ** -9).astype(np.int64)
    nrm = ~sub
    _, ve = np.frexp(value[nrm])
    ev = (ve - 1).astype(np.int64)
    mant = np.rint((value[nrm] / np.exp2(ev.astype(np.float64)) - 1.0) * 8.0).astype(np.int64)
    code[nrm] = ((ev + 7) << 3) | mant
    return (code | np.where(sign, 0x80, 0)).astype(np.uint8)


def quantize(x: np.ndarray, scale: float) -> np.ndarray:
    """Static-scale quantization: E4M3 codes of x * r, the product in float32, where the scale
    is a float32 and r is its reciprocal rounded to float32."""
    s = float(np.float32(scale))
    inv = np.float32(1.0 / s)
    return e4m3_encode(np.asarray(x, dtype=np.float32) * inv)


def dequantize(codes: np.ndarray, scale: float) -> np.ndarray:
    """Values code * scale in float64, the scale taken as a float32."""
    return e4m3_decode(codes) * float(np.float32(scale))


def attention_q_scale(q_scale: float, k_scale: float, head_dim: int) -> float:
    """The scale q is quantized with for attention (float32, returned as a Python float).

    With c = log2(e)/sqrt(head_dim) and the float32 scales, x = c * q_scale * k_scale; the
    exponent e = ceil(log2 x) (x = f 2^e' with f in [0.5, 1) from frexp: e = e' - 1 when f is
    exactly 0.5, else e'); the result is float32(2^e / (c * k_scale)), i.e. the smallest
    q_scale' >= q_scale (up to that rounding) with c * q_scale' * k_scale a power of two.
    Every step is taken in float64 from the float32 scales."""
    c = 1.4426950408889634 / math.sqrt(head_dim)
    ks = float(np.float32(k_scale))
    x = c * float(np.float32(q_scale)) * ks
    f, e = math.frexp(x)
    if f == 0.5:
        e -= 1
    return float(np.float32(math.ldexp(1.0, e) / (c * ks)))
