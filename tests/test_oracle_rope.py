"""Pins for oracle/rope.py: closed forms, invariants, brute force, negative control."""

import json
import math
import os

import numpy as np
import pytest

from oracle import rope as P
from oracle import rounding as R
from oracle.brute import (FMT_BF16, FMT_F16, FMT_F32, brute_rotate_def,
                          brute_rotate_method, round_fraction)

from conftest import GOLDEN

FACTS = json.load(open(os.path.join(GOLDEN, "pages_facts.json")))


def test_theta_closed_forms():
    th = P.rope_frequencies(64, 10000.0)
    assert th.shape == (32,)
    assert th[0] == 1.0                       # the fastest pair turns 1 rad per position
    assert abs(th[16] - 0.01) < 1e-17         # 10000^(-1/2)
    assert abs(th[31] / 10 ** -3.875 - 1) < 1e-14
    # strictly decreasing geometric sequence with ratio base^(-2/D)
    ratio = th[1:] / th[:-1]
    assert np.allclose(ratio, 10000.0 ** (-2 / 64), rtol=1e-14, atol=0)


def test_position_zero_is_identity():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((1, 64))
    c, s = np.cos(P.rope_angles(1, 64)), np.sin(P.rope_angles(1, 64))
    np.testing.assert_array_equal(P.rotate_def(x, c, s), x)
    c32, s32 = P.rope_table_f32(1, 64)
    for io in ("f16", "bf16"):
        xi = R.round_io(x.astype(np.float32), io)
        np.testing.assert_array_equal(P.rotate_method(xi, c32, s32, io), xi)


def test_d2_rotates_by_m_radians():
    L = 50
    x = np.zeros((L, 2))
    x[:, 0] = 1.0
    phi = P.rope_angles(L, 2)
    assert np.array_equal(phi[:, 0], np.arange(L, dtype=float))
    r = P.rotate_def(x, np.cos(phi), np.sin(phi))
    m = np.arange(L)
    np.testing.assert_allclose(r[:, 0], np.cos(m), rtol=0, atol=1e-15)
    np.testing.assert_allclose(r[:, 1], np.sin(m), rtol=0, atol=1e-15)
    # a (0, 1) vector rotates the other way round: (-sin, cos)
    y = np.zeros((L, 2))
    y[:, 1] = 1.0
    r = P.rotate_def(y, np.cos(phi), np.sin(phi))
    np.testing.assert_allclose(r[:, 0], -np.sin(m), rtol=0, atol=1e-15)
    np.testing.assert_allclose(r[:, 1], np.cos(m), rtol=0, atol=1e-15)


def test_pair_norm_preserved():
    rng = np.random.default_rng(1)
    L, D = 300, 64
    x = rng.standard_normal((2, L, D))
    phi = P.rope_angles(L, D)
    r = P.rotate_def(x, np.cos(phi), np.sin(phi))
    n0 = x[..., 0::2] ** 2 + x[..., 1::2] ** 2
    n1 = r[..., 0::2] ** 2 + r[..., 1::2] ** 2
    assert np.max(np.abs(n1 / n0 - 1)) < 1e-12


def _rot_at(x, m, D, base=10000.0):
    th = P.rope_frequencies(D, base)
    phi = m * th
    return P.rotate_def(x[None, :], np.cos(phi)[None, :], np.sin(phi)[None, :])[0]


def test_dot_depends_only_on_offset():
    rng = np.random.default_rng(2)
    D = 64
    for _ in range(200):
        q, k = rng.standard_normal(D), rng.standard_normal(D)
        m, n, t = (int(v) for v in rng.integers(0, 8192, 3))
        a = _rot_at(q, m, D) @ _rot_at(k, n, D)
        b = _rot_at(q, m + t, D) @ _rot_at(k, n + t, D)
        assert abs(a - b) < 1e-9 * (1 + abs(a))


def test_table_is_one_rounding_of_fp64_trig():
    L, D = 4096, 64
    c32, s32 = P.rope_table_f32(L, D)
    assert c32.dtype == np.float32 and c32.shape == (L, D // 2)
    rng = np.random.default_rng(3)
    th = [10000.0 ** (-2.0 * i / D) for i in range(D // 2)]
    for _ in range(3000):
        m, i = int(rng.integers(0, L)), int(rng.integers(0, D // 2))
        phi = float(m) * th[i]
        assert float(c32[m, i]) == float(round_fraction(math.cos(phi), FMT_F32))
        assert float(s32[m, i]) == float(round_fraction(math.sin(phi), FMT_F32))


def test_rotate_def_matches_brute():
    rng = np.random.default_rng(4)
    for D in (2, 4, 8, 64):
        L = 12
        x = rng.standard_normal((L, D))
        phi = P.rope_angles(L, D)
        got = P.rotate_def(x, np.cos(phi), np.sin(phi))
        want = np.array(brute_rotate_def(x.tolist(), D, 10000.0))
        np.testing.assert_allclose(got, want, rtol=0, atol=1e-13)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("io,fmt", [("f16", FMT_F16), ("bf16", FMT_BF16)])
def test_rotate_method_bit_exact_vs_rational(io, fmt, D):
    rng = np.random.default_rng(5 + D)
    L = 40
    # large positions too, where fp32 table values are irregular
    pos = np.concatenate([np.arange(20), rng.integers(20, 8192, 20)])
    c32, s32 = P.rope_table_f32(8192, D)
    c32, s32 = c32[pos], s32[pos]
    x = R.round_io((rng.standard_normal((L, D)) * 2).astype(np.float32), io)
    got = P.rotate_method(x, c32, s32, io)
    want = np.array(brute_rotate_method(x.tolist(), c32.astype(float).tolist(),
                                        s32.astype(float).tolist(), fmt))
    np.testing.assert_array_equal(got, want)


def test_rotate_f32_bit_exact_vs_rational():
    """The FP32 stage itself, before the cast: a fused or reordered rotation differs here."""
    rng = np.random.default_rng(9)
    L, D = 64, 64
    pos = rng.integers(0, 8192, L)
    c32, s32 = P.rope_table_f32(8192, D)
    c32, s32 = c32[pos], s32[pos]
    x = R.round_io((rng.standard_normal((L, D)) * 3).astype(np.float32), "bf16")
    got = P.rotate_f32(x, c32, s32)
    assert got.dtype == np.float32
    want = np.array(brute_rotate_method(x.tolist(), c32.astype(float).tolist(),
                                        s32.astype(float).tolist(), None))
    np.testing.assert_array_equal(got.astype(np.float64), want)


def test_bf16_angle_spacing_matches_pages():
    fact = FACTS["bf16_angle_spacing"]
    a = np.float32(fact["angle_rad"])
    bits = R.f32_to_bf16_bits(np.array([a]))
    lo = R.bf16_bits_to_f64(bits)[0]
    hi = R.bf16_bits_to_f64(bits + 1)[0]
    assert hi - lo == fact["spacing_rad"]
    assert hi - lo > 2 * math.pi


def test_negative_control_bf16_angle_breaks_relative_position():
    """A bf16-evaluated angle destroys position information at long L; FP32 keeps it."""
    L, D = 4096, 64
    c32, s32 = P.rope_table_f32(L, D)
    cb, sb, phi_bf = P.rope_table_bf16_angle(L, D)
    rng = np.random.default_rng(6)
    q, k = rng.standard_normal(D), rng.standard_normal(D)

    def dot(c, s, m, n):
        qm = P.rotate_def(q[None], c[m:m + 1], s[m:m + 1])[0]
        kn = P.rotate_def(k[None], c[n:n + 1], s[n:n + 1])[0]
        return qm @ kn

    err32, errbf = 0.0, 0.0
    for _ in range(100):
        m, n = (int(v) for v in rng.integers(0, 64, 2))
        t = int(rng.integers(3500, L - 64))
        err32 = max(err32, abs(dot(c32, s32, m, n) - dot(c32, s32, m + t, n + t)))
        errbf = max(errbf, abs(dot(cb, sb, m, n) - dot(cb, sb, m + t, n + t)))
    assert err32 < 1e-4
    assert errbf > 1.0


# ---- RoPE options: half-split pairing and partial rotary width -------------------

ROTARY = [(16, "adjacent"), (32, "adjacent"), (48, "adjacent"), (16, "half"), (32, "half"), (48, "half"),
          (64, "half")]


def _half_to_adjacent(x, rd):
    """Permutation taking half-split pair members to adjacent slots: y[2i] = x[i],
    y[2i+1] = x[i + rd/2] for i < rd/2; dims >= rd in place."""
    y = np.array(x, copy=True)
    y[..., 0:rd:2] = x[..., :rd // 2]
    y[..., 1:rd:2] = x[..., rd // 2:rd]
    return y


@pytest.mark.parametrize("rd", [16, 32, 48, 64])
def test_half_split_is_adjacent_on_permuted_dims(rd):
    """The half-split FP32 rotation is the adjacent one applied to permuted dims, bit
    for bit: the same FP32 operations on the same operand pairs."""
    rng = np.random.default_rng(20 + rd)
    L, D = 50, 64
    pos = rng.integers(0, 8192, L)
    c32, s32 = P.rope_table_f32(8192, rd)
    c32, s32 = c32[pos], s32[pos]
    x = R_round((rng.standard_normal((L, D)) * 3))
    got = P.rotate_f32(x, c32, s32, pairing="half", rotary_dim=rd)
    want = P.rotate_f32(_half_to_adjacent(x, rd), c32, s32, rotary_dim=rd)
    np.testing.assert_array_equal(_half_to_adjacent(got, rd), want)


def R_round(x):
    return R.round_io(np.asarray(x, dtype=np.float32), "bf16")


@pytest.mark.parametrize("rd,pairing", ROTARY)
def test_partial_rotary_leaves_the_tail_and_rotates_the_head(rd, pairing):
    rng = np.random.default_rng(30 + rd)
    L, D = 40, 64
    c32, s32 = P.rope_table_f32(L, rd)
    x = R_round(rng.standard_normal((L, D)) * 2)
    got = P.rotate_f32(x, c32, s32, pairing=pairing, rotary_dim=rd)
    # trailing dims are the input, exactly
    np.testing.assert_array_equal(got[:, rd:].astype(np.float64), x[:, rd:])
    # leading dims are the full-width rotation of a head of dim rd
    head = P.rotate_f32(x[:, :rd], c32, s32, pairing=pairing)
    np.testing.assert_array_equal(got[:, :rd], head)


# head dim 128: rotary widths past 64, and the full width
ROTARY_128 = [(96, "adjacent"), (96, "half"), (112, "half"), (128, "half"), (128, "adjacent")]


@pytest.mark.parametrize("rd,pairing,D", [(r, p, 64) for r, p in ROTARY + [(64, "adjacent")]] +
                         [(r, p, 128) for r, p in ROTARY_128] + [(32, "half", 128)])
@pytest.mark.parametrize("io,fmt", [("f16", FMT_F16), ("bf16", FMT_BF16)])
def test_rotation_options_bit_exact_vs_rational(rd, pairing, D, io, fmt):
    rng = np.random.default_rng(40 + rd + D)
    L = 24
    pos = np.concatenate([np.arange(8), rng.integers(8, 8192, 16)])
    c32, s32 = P.rope_table_f32(8192, rd)
    c32, s32 = c32[pos], s32[pos]
    x = R.round_io((rng.standard_normal((L, D)) * 2).astype(np.float32), io)
    got = P.rotate_method(x, c32, s32, io, pairing=pairing, rotary_dim=rd)
    want = np.array(brute_rotate_method(x.tolist(), c32.astype(float).tolist(), s32.astype(float).tolist(),
                                        fmt, pairing=pairing, rotary_dim=rd))
    np.testing.assert_array_equal(got, want)


@pytest.mark.parametrize("rd,pairing,D", [(r, p, 64) for r, p in ROTARY] + [(r, p, 128) for r, p in ROTARY_128])
def test_rotate_def_options_match_brute(rd, pairing, D):
    rng = np.random.default_rng(50 + rd + D)
    L = 12
    x = rng.standard_normal((L, D))
    phi = P.rope_angles(L, rd)
    got = P.rotate_def(x, np.cos(phi), np.sin(phi), pairing=pairing, rotary_dim=rd)
    want = np.array(brute_rotate_def(x.tolist(), D, 10000.0, pairing=pairing, rotary_dim=rd))
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-13)


@pytest.mark.parametrize("rd,pairing", ROTARY)
def test_dot_depends_only_on_offset_with_options(rd, pairing):
    rng = np.random.default_rng(60 + rd)
    D = 64
    th = P.rope_frequencies(rd)

    def rot(x, m):
        phi = m * th
        return P.rotate_def(x[None, :], np.cos(phi)[None, :], np.sin(phi)[None, :], pairing=pairing,
                            rotary_dim=rd)[0]

    for _ in range(100):
        q, k = rng.standard_normal(D), rng.standard_normal(D)
        m, n, t = (int(v) for v in rng.integers(0, 8192, 3))
        a, b = rot(q, m) @ rot(k, n), rot(q, m + t) @ rot(k, n + t)
        assert abs(a - b) < 1e-9 * (1 + abs(a))


def test_rotation_option_errors():
    x = np.zeros((2, 64))
    c, s = P.rope_table_f32(2, 64)
    with pytest.raises(ValueError):
        P.rotate_f32(x, c, s, pairing="interleaved")
    with pytest.raises(ValueError):
        P.rotate_f32(x, c, s, rotary_dim=66)
    with pytest.raises(ValueError):
        P.rotate_f32(x, c, s, rotary_dim=15)
