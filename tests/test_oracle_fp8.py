"""Pins for the oracle's number formats (CPU only).

The fp8 codec is checked against the OCP E4M3 definition's landmark values
and against PyTorch's CPU float8_e4m3fn cast (a library routine) on every
code, every midpoint and random values; bf16 rounding against PyTorch's
float32 -> bfloat16 cast; the UE8M0 round-up rule against the closed form
clip(ceil(log2 s) + 127, 0, 254) computed with frexp.
"""

import numpy as np
import pytest
import torch

from oracle import fp8


def torch_e4m3(values):
    t = torch.from_numpy(np.asarray(values, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_decode_landmarks():
    # Values fixed by the format definition (bias 7, 3 mantissa bits).
    assert fp8.decode_e4m3(0x7E) == 448.0            # largest finite
    assert fp8.decode_e4m3(0x38) == 1.0
    assert fp8.decode_e4m3(0x08) == 2.0 ** -6        # smallest normal
    assert fp8.decode_e4m3(0x01) == 2.0 ** -9        # smallest subnormal
    assert fp8.decode_e4m3(0x07) == 7 * 2.0 ** -9    # largest subnormal
    assert fp8.decode_e4m3(0xB8) == -1.0
    assert np.isnan(fp8.decode_e4m3(0x7F)) and np.isnan(fp8.decode_e4m3(0xFF))
    assert fp8.decode_e4m3(0x80) == 0.0 and np.signbit(fp8.decode_e4m3(0x80))


def test_decode_matches_torch_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy()
    ours = fp8.decode_e4m3(codes)
    both_nan = np.isnan(ref) & np.isnan(ours)
    assert np.all(both_nan | (ref == ours))
    assert np.array_equal(np.signbit(ref[~both_nan]), np.signbit(ours[~both_nan]))


def test_encode_roundtrip_all_finite_codes():
    codes = np.arange(256, dtype=np.uint8)
    vals = fp8.decode_e4m3(codes)
    fin = ~np.isnan(vals)
    assert np.array_equal(fp8.encode_e4m3(vals[fin]), codes[fin])


def test_encode_midpoints_ties_to_even_match_torch():
    pos = np.sort(fp8.decode_e4m3(np.arange(0x00, 0x7F, dtype=np.uint8)))
    mids = (pos[:-1] + pos[1:]) / 2.0           # exact in float32
    vals = np.concatenate([mids, -mids, mids * (1 + 2 ** -20), mids * (1 - 2 ** -20)])
    assert np.array_equal(fp8.encode_e4m3(vals.astype(np.float32)),
                          torch_e4m3(vals))
    # Ties go to the even mantissa: between 1.0 (0x38) and 1.125 (0x39).
    assert fp8.encode_e4m3(1.0625) == 0x38
    assert fp8.encode_e4m3(1.1875) == 0x3A


def test_encode_random_matches_torch():
    rng = np.random.default_rng(7)
    vals = np.concatenate([
        rng.uniform(-460, 460, 200000),
        rng.standard_normal(200000) * 2.0 ** rng.integers(-12, 8, 200000),
        rng.uniform(-2 ** -6, 2 ** -6, 50000),
    ]).astype(np.float32)
    assert np.array_equal(fp8.encode_e4m3(vals), torch_e4m3(vals))


def test_encode_float64_path_agrees_and_rounds_once():
    # Values exactly representable in float32 take the same code on both paths;
    # values a hair above or below a midpoint (not float32 numbers) round once.
    rng = np.random.default_rng(8)
    v32 = (rng.uniform(-470, 470, 100000)).astype(np.float32)
    assert np.array_equal(fp8.encode_e4m3(v32), fp8.encode_e4m3(v32.astype(np.float64)))
    pos = np.sort(fp8.decode_e4m3(np.arange(0x00, 0x7F, dtype=np.uint8)))
    mids = (pos[:-1] + pos[1:]) / 2.0
    up = fp8.encode_e4m3(mids * (1 + 2.0 ** -40))
    down = fp8.encode_e4m3(mids * (1 - 2.0 ** -40))
    assert np.array_equal(up, np.arange(1, 0x7F, dtype=np.uint8))
    assert np.array_equal(down[1:], np.arange(1, 0x7E, dtype=np.uint8))


def test_encode_overflow_and_specials():
    # 464 is the tie between 448 and the NaN slot: ties to even gives 448;
    # anything above rounds past 448 and this non-saturating encoder gives NaN.
    assert fp8.encode_e4m3(464.0) == 0x7E
    assert fp8.encode_e4m3(464.5) == 0x7F
    assert fp8.encode_e4m3(-500.0) == 0xFF
    assert fp8.encode_e4m3(np.nan) & 0x7F == 0x7F
    assert fp8.encode_e4m3(np.inf) == 0x7F
    assert fp8.encode_e4m3(-0.0) == 0x80
    assert fp8.encode_e4m3(2.0 ** -10) == 0x00          # tie with 2^-9: to even (0)
    assert fp8.encode_e4m3(2.0 ** -10 * 1.01) == 0x01
    np.testing.assert_array_equal(
        fp8.encode_e4m3(np.array([464.0, 500.0, -0.0, 2 ** -10], np.float32)),
        torch_e4m3([464.0, 500.0, -0.0, 2 ** -10]))


def test_round_bf16_matches_torch():
    rng = np.random.default_rng(3)
    v = (rng.standard_normal(500000) * 2.0 ** rng.integers(-30, 30, 500000)).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.bfloat16).float().numpy()
    assert np.array_equal(fp8.round_bf16(v), ref)
    # Ties to even at the bf16 lsb (2^-7 at 1.0).
    assert fp8.round_bf16(1.0 + 2 ** -8) == 1.0
    assert fp8.round_bf16(1.0 + 3 * 2 ** -8) == 1.0 + 2 ** -6
    # Single rounding from float64: just above the tie goes up.
    assert fp8.round_bf16(1.0 + 2 ** -8 + 2 ** -40) == 1.0 + 2 ** -7


def test_bf16_bits_roundtrip():
    v = fp8.round_bf16(np.linspace(-3, 3, 101))
    assert np.array_equal(fp8.bf16_from_bits(fp8.bf16_bits(v)), v)


def _e8m0_closed_form(s):
    s = np.asarray(s, dtype=np.float32).astype(np.float64)
    f, ex = np.frexp(s)
    c = np.where(f == 0.5, ex - 1, ex).astype(np.int64)   # ceil(log2 s)
    c = np.where(s == 0, -1000, c)
    return np.clip(c + 127, 0, 254).astype(np.uint8)


def test_e8m0_round_up_closed_form():
    rng = np.random.default_rng(11)
    s = np.concatenate([
        (rng.uniform(0.5, 1.0, 100000) * 2.0 ** rng.integers(-140, 128, 100000)),
        2.0 ** np.arange(-149, 128, dtype=np.float64),
    ]).astype(np.float32)
    s = s[np.isfinite(s)]
    assert np.array_equal(fp8.e8m0_round_up(s), _e8m0_closed_form(s))


@pytest.mark.parametrize("bits,expect", [
    (0x3F800000, 127),          # 1.0: exact power of two stays
    (0x3F800001, 128),          # one ulp above 1.0 rounds up
    (0x3FFFFFFF, 128),          # just below 2.0
    (0x7F000000, 254),          # 2^127 exact
    (0x7F000001, 254),          # exponent field 0xFE is never bumped
    (0x00400000, 0),            # subnormal 2^-127: byte 0 already bounds it
    (0x00400001, 1),            # just above 2^-127 -> 2^-126
    (0x00000001, 0),            # smallest subnormal
    (0x00000000, 0),            # zero
])
def test_e8m0_edges(bits, expect):
    s = np.array([bits], dtype=np.uint32).view(np.float32)
    assert int(fp8.e8m0_round_up(s)[0]) == expect
    if (bits >> 23) != 0xFE:        # the top binade cannot be rounded up
        assert fp8.e8m0_value(expect) >= s[0]
