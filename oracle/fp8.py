"""OCP FP8 E4M3 ("fn" variant) codec, written from the format definition.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

[P2], section "vLLM 也不是银弹：真实部署中的坑" (third pitfall) names an FP8
KV cache as the way to shrink long-context KV memory, and fixes nothing else.
Readings taken where the page is silent:

* the format is OCP E4M3 "fn": 1 sign bit, 4 exponent bits with bias 7,
  3 mantissa bits; exponent field 0 holds subnormals m * 2^-9; the only NaN
  codes are S.1111.111 (0x7F, 0xFF); there are no infinities; the largest
  finite magnitude is 448;
* encoding takes a float32 value, rounds it to the nearest finite E4M3 value
  with ties going to the code whose mantissa is even, saturates magnitudes
  above 448 to 448, and keeps the sign (so tiny negatives become 0x80);
* a cached element is encode(fp32(x / scale)) with one fp32 scale per KV
  head, and its value is decode(code) * scale.
"""

import numpy as np

E4M3_MAX = 448.0


def e4m3_value(code: int) -> float:
    """Value of one E4M3 code, straight from the bit-field definition."""
    sign = -1.0 if code & 0x80 else 1.0
    exp_field = (code >> 3) & 0xF
    mant = code & 0x7
    if exp_field == 0xF and mant == 0x7:
        return float("nan")
    if exp_field == 0:
        return sign * mant * 2.0 ** -9
    return sign * (1.0 + mant / 8.0) * 2.0 ** (exp_field - 7)


# 256-entry decode table (float64; every E4M3 value is exact in float64).
E4M3_TABLE = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)

# Codes 0x00..0x7E are the non-negative finite values in increasing order.
_POSITIVE = E4M3_TABLE[:0x7F].copy()


def e4m3_decode(codes) -> np.ndarray:
    """Decode uint8 codes to float64 values (NaN for 0x7F / 0xFF)."""
    return E4M3_TABLE[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode(x) -> np.ndarray:
    """Encode float32 values: nearest finite E4M3, ties to even code, saturate.

    The nearest value is found by searching the sorted table of non-negative
    finite values, so the rounding is the definition itself rather than a
    bit manipulation. All distances are exact in float64.
    """
    x = np.asarray(x, dtype=np.float32).astype(np.float64)
    negative = np.signbit(x)
    mag = np.minimum(np.abs(x), E4M3_MAX)
    hi = np.searchsorted(_POSITIVE, mag, side="left")
    hi = np.minimum(hi, 0x7E)
    lo = np.maximum(hi - 1, 0)
    d_hi = _POSITIVE[hi] - mag
    d_lo = mag - _POSITIVE[lo]
    take_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(take_hi, hi, lo).astype(np.uint16)
    code = np.where(np.isnan(x), 0x7F, code)
    code = code | (negative.astype(np.uint16) << 7)
    return code.astype(np.uint8)


def quotient_f32(x_f64, scale_f32) -> np.ndarray:
    """fp32(x / scale): the float64 quotient rounded once to float32.

    x holds fp16/bf16 values (exact in float64) and scale is an fp32 value,
    so the float64 quotient rounded to float32 is the correctly rounded fp32
    quotient (double rounding through a 53-bit format is harmless for a
    24-bit division).
    """
    x = np.asarray(x_f64, dtype=np.float64)
    s = np.asarray(scale_f32, dtype=np.float32).astype(np.float64)
    return (x / s).astype(np.float32)


def quantize(x_f64, scale_f32) -> np.ndarray:
    """Stored code of a source value x under one per-head fp32 scale."""
    return e4m3_encode(quotient_f32(x_f64, scale_f32))


def dequantize(codes, scale_f32) -> np.ndarray:
    """Value of a stored code under its per-head fp32 scale, in float64.

    decode(code) has at most a 4-bit significand and the scale a 24-bit one,
    so the float64 product is exact.
    """
    s = np.asarray(scale_f32, dtype=np.float32).astype(np.float64)
    return e4m3_decode(codes) * s
