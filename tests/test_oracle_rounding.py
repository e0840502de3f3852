"""Pins for oracle/rounding.py: every cast checked against exact rational RNE.

The reference rounding is oracle/brute.round_fraction, written with
fractions.Fraction independently of the numpy code under test.
"""

import math
import struct

import numpy as np
import pytest

from oracle import rounding as R
from oracle.brute import FMT_BF16, FMT_F16, FMT_F32, round_fraction


def _f32_values(n, seed):
    """fp32 values spread over many exponents, plus exact ties and specials."""
    rng = np.random.default_rng(seed)
    bits = rng.integers(0, 2**32, size=n, dtype=np.uint64).astype(np.uint32)
    # keep exponents mostly in a sane band but include subnormal and huge ones
    exp = rng.integers(0, 255, size=n).astype(np.uint32)
    bits = (bits & np.uint32(0x807FFFFF)) | (exp << np.uint32(23))
    x = bits.view(np.float32).copy()
    x = x[np.isfinite(x)]
    return x


def _bf16_ties():
    rng = np.random.default_rng(7)
    hi = rng.integers(0, 0x7F7F, size=2000).astype(np.uint32)
    bits = (hi << np.uint32(16)) | np.uint32(0x8000)  # exactly halfway
    bits = np.concatenate([bits, bits | np.uint32(0x80000000)])
    return bits.view(np.float32)


def _f16_ties():
    # fp32 values exactly halfway between adjacent fp16 normals and subnormals
    rng = np.random.default_rng(8)
    out = []
    for _ in range(3000):
        e = int(rng.integers(-24, 16))
        m = int(rng.integers(0, 1 << 11))
        # value = (m + 0.5) * 2^(e-10) lies halfway on the fp16 grid of exponent e
        v = (m + 0.5) * 2.0 ** (e - 10)
        if v < 65504:
            out.append(v)
            out.append(-v)
    return np.array(out, dtype=np.float32)


def _as_frac_rounded(x, fmt):
    r = round_fraction(float(x), fmt)
    return r if isinstance(r, float) else float(r)


def test_bf16_matches_exact_rne_random():
    x = _f32_values(20000, 1)
    got = R.bf16_bits_to_f64(R.f32_to_bf16_bits(x))
    want = np.array([_as_frac_rounded(v, FMT_BF16) for v in x])
    np.testing.assert_array_equal(got, want)


def test_bf16_ties_round_to_even():
    x = _bf16_ties()
    got = R.bf16_bits_to_f64(R.f32_to_bf16_bits(x))
    want = np.array([_as_frac_rounded(v, FMT_BF16) for v in x])
    np.testing.assert_array_equal(got, want)
    # the kept significand is even after a tie
    bits = R.f32_to_bf16_bits(x)
    assert np.all((bits & 1) == 0)


def test_bf16_specials():
    x = np.array([0.0, -0.0, np.inf, -np.inf, np.float32(3.4028235e38), np.float32(1e-45)], dtype=np.float32)
    got = R.bf16_bits_to_f64(R.f32_to_bf16_bits(x))
    assert got[0] == 0 and got[1] == 0 and math.copysign(1, got[1]) == -1
    assert got[2] == np.inf and got[3] == -np.inf
    assert got[4] == np.inf  # largest fp32 lies above the bf16 overflow midpoint
    assert got[5] == 0.0     # smallest subnormal rounds to zero in bf16
    nan = R.f32_to_bf16_bits(np.array([np.nan], dtype=np.float32))
    assert np.isnan(R.bf16_bits_to_f64(nan))[0]


def test_f16_matches_exact_rne():
    x = _f32_values(20000, 2)
    x = x[np.abs(x) < 1e6]
    x = np.concatenate([x, _f16_ties(), np.array([65504, 65519.99, 65520, 1e-8, 2.0**-24, 2.0**-25, 3 * 2.0**-26], dtype=np.float32)])
    got = R.f32_to_f16(x).astype(np.float64)
    want = np.array([_as_frac_rounded(v, FMT_F16) for v in x])
    np.testing.assert_array_equal(got, want)


def test_f32_matches_exact_rne():
    rng = np.random.default_rng(3)
    x = rng.standard_normal(5000) * np.exp(rng.uniform(-80, 80, 5000))
    got = R.f32(x).astype(np.float64)
    want = np.array([_as_frac_rounded(v, FMT_F32) for v in x])
    np.testing.assert_array_equal(got, want)
    # struct's fp32 packing is an independent third opinion
    via_struct = np.array([struct.unpack("f", struct.pack("f", v))[0] for v in x])
    np.testing.assert_array_equal(got, via_struct)


@pytest.mark.parametrize("io", ["f16", "bf16"])
def test_round_io_is_idempotent_and_widen_exact(io):
    rng = np.random.default_rng(4)
    x = rng.standard_normal(4000).astype(np.float32)
    once = R.round_io(x, io)
    twice = R.round_io(once.astype(np.float32), io)
    np.testing.assert_array_equal(once, twice)
