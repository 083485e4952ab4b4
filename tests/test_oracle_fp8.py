"""Pins of the oracle's E4M3 codec.

Pinned against: the format definition's landmark values (worked by hand),
torch's float8_e4m3fn conversions (a library routine) over every code and
over every finite fp16 input in range, and hand-worked tie and saturation
cases.
"""

import math

import numpy as np
import pytest
import torch

from oracle import fp8


def check_decode_table(decode):
    codes = np.arange(256, dtype=np.uint8)
    ours = decode(codes)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan_ours = np.isnan(ours)
    assert np.array_equal(nan_ours, np.isnan(ref))
    assert np.array_equal(np.flatnonzero(nan_ours), [0x7F, 0xFF])
    assert np.array_equal(ours[~nan_ours], ref[~nan_ours])
    # Signs of zeros too.
    assert np.array_equal(np.signbit(ours[~nan_ours]), np.signbit(ref[~nan_ours]))


def test_decode_table_matches_torch():
    check_decode_table(fp8.e4m3_decode)


def test_decode_landmarks_from_format_definition():
    d = fp8.e4m3_decode
    assert d(0x00) == 0.0 and np.signbit(d(0x80))
    assert d(0x01) == 2.0 ** -9            # smallest subnormal
    assert d(0x07) == 7 * 2.0 ** -9        # largest subnormal
    assert d(0x08) == 2.0 ** -6            # smallest normal
    assert d(0x38) == 1.0
    assert d(0x39) == 1.125
    assert d(0x7E) == 448.0 == fp8.E4M3_MAX
    assert d(0xFE) == -448.0
    assert math.isnan(d(0x7F)) and math.isnan(d(0xFF))
    pos = fp8.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    assert np.all(np.diff(pos) > 0)


def check_encoder_against_torch(encode):
    """Every finite fp16 value, divided by several scales, inside +-448."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    x = bits.view(np.float16).astype(np.float64)
    x = x[np.isfinite(x)]
    for scale in (1.0, 0.5, 0.011, 1.0 / 448.0, 3.7, 2.0 ** -7, 123.25):
        s32 = np.float32(scale)
        q = fp8.quotient_f32(x, s32)
        keep = np.abs(q.astype(np.float64)) <= 448.0
        q = q[keep]
        ours = encode(q)
        ref = torch.from_numpy(q.copy()).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert np.array_equal(ours, ref), f"scale {scale}"


def test_encoder_matches_torch_in_range():
    check_encoder_against_torch(fp8.e4m3_encode)


def check_ties_and_saturation(encode):
    f = lambda v: int(encode(np.float32(v)))  # noqa: E731
    # ties go to the even code
    assert f(1.0625) == 0x38          # between 1.0 (0x38) and 1.125 (0x39)
    assert f(1.1875) == 0x3A          # between 1.125 (0x39) and 1.25 (0x3A)
    assert f(2.0 ** -10) == 0x00      # half the smallest subnormal
    assert f(3 * 2.0 ** -10) == 0x02  # between 2^-9 (0x01) and 2^-8 (0x02)
    assert f(-1.0625) == 0xB8
    # just off a tie
    assert f(np.nextafter(np.float32(1.0625), np.float32(2))) == 0x39
    # saturation keeps the sign and never yields NaN for finite input
    for v in (448.0, 449.0, 463.9, 464.0, 480.0, 1e6, 3.0e38, float("inf")):
        assert f(v) == 0x7E and f(-v) == 0xFE
    assert f(0.0) == 0x00 and f(-0.0) == 0x80
    assert f(-1e-30) == 0x80


def test_ties_and_saturation():
    check_ties_and_saturation(fp8.e4m3_encode)


def test_encode_decode_round_trip_all_finite_codes():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = fp8.e4m3_decode(codes).astype(np.float32)
    assert np.array_equal(fp8.e4m3_encode(vals), codes)


def test_rounding_error_bound():
    """|dequant - x/s| is at most half a code spacing (2^-4 relative for
    normals, 2^-10 absolute for subnormals)."""
    rng = np.random.default_rng(1)
    x = rng.standard_normal(200_000) * 50
    q = fp8.quotient_f32(x, np.float32(1.0))
    back = fp8.e4m3_decode(fp8.e4m3_encode(q))
    qd = q.astype(np.float64)
    inside = np.abs(qd) <= 448
    err = np.abs(back - qd)[inside]
    bound = np.maximum(np.abs(qd)[inside] * 2.0 ** -4, 2.0 ** -10)
    assert np.all(err <= bound)


def test_quotient_is_correctly_rounded_fp32_division():
    rng = np.random.default_rng(2)
    x = rng.standard_normal(10000).astype(np.float16).astype(np.float64)
    s = np.float32(0.0123)
    q = fp8.quotient_f32(x, s)
    t = torch.from_numpy(x.astype(np.float32)) / torch.tensor(s, dtype=torch.float32)
    assert np.array_equal(q, t.numpy())


def test_dequantize_is_exact_product():
    codes = np.arange(0x7F, dtype=np.uint8)
    s = np.float32(0.0037)
    ref = np.array([fp8.e4m3_value(int(c)) for c in codes]) * float(s)
    assert np.array_equal(fp8.dequantize(codes, s), ref)


@pytest.mark.parametrize("bad", ["ties_away", "no_saturation"])
def test_planted_codec_mistakes_are_caught(bad):
    """A plausible mistake in the encoder fails one of the pins above."""
    positive = fp8.e4m3_decode(np.arange(0x7F, dtype=np.uint8))

    def ties_away(x):
        x = np.asarray(x, dtype=np.float32).astype(np.float64)
        mag = np.minimum(np.abs(x), 448.0)
        hi = np.minimum(np.searchsorted(positive, mag), 0x7E)
        lo = np.maximum(hi - 1, 0)
        code = np.where(positive[hi] - mag <= mag - positive[lo], hi, lo)
        return (code | (np.signbit(x) << 7)).astype(np.uint8)

    def no_saturation(x):
        x = np.asarray(x, dtype=np.float32).astype(np.float64)
        big = np.abs(x) > 464
        out = fp8.e4m3_encode(x)
        return np.where(big, out | 0x7F, out).astype(np.uint8)

    impl = {"ties_away": ties_away, "no_saturation": no_saturation}[bad]
    with pytest.raises(AssertionError):
        check_ties_and_saturation(impl)
