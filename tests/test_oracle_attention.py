"""Pins for oracle/attention.py: brute force, invariants, closed forms, page facts."""

import json
import os

import numpy as np
import pytest

from oracle import attention as A
from oracle import rope as P
from oracle import rounding as R
from oracle.brute import FMT_BF16, FMT_F16, brute_attention

from conftest import GOLDEN

FACTS = json.load(open(os.path.join(GOLDEN, "pages_facts.json")))


def _rand(shape, seed, io=None):
    x = np.random.default_rng(seed).standard_normal(shape)
    if io is not None:
        x = R.round_io(x.astype(np.float32), io)
    return x


CASES = [(L, D, w) for L in (1, 2, 3, 5, 8, 12) for D in (2, 4, 8)
         for w in sorted({-1, 0, 1, 2, max(L - 1, 0), L})]


@pytest.mark.parametrize("L,D,w", CASES)
def test_def_mode_matches_brute(L, D, w):
    q, k, v = (_rand((1, 1, L, D), s) for s in (10 + L, 20 + D, 30 + w))
    scale = 1 / np.sqrt(D) * 1.7
    got = A.attn_def(q, k, v, scale, window=w)[0, 0]
    want = np.array(brute_attention(q[0, 0].tolist(), k[0, 0].tolist(), v[0, 0].tolist(), scale, w))
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


@pytest.mark.parametrize("lam", [0.0, 0.8, -0.3])
@pytest.mark.parametrize("w", [-1, 0, 2, 11])
def test_def_mode_differential_matches_brute(lam, w):
    L, D = 12, 8
    q, k, q2, k2, v = (_rand((1, 1, L, D), s) for s in range(40, 45))
    scale = 0.4
    got = A.attn_def(q, k, v, scale, window=w, lam=lam, q2=q2, k2=k2)[0, 0]
    want = np.array(brute_attention(q[0, 0].tolist(), k[0, 0].tolist(), v[0, 0].tolist(),
                                    scale, w, lam, q2[0, 0].tolist(), k2[0, 0].tolist()))
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


@pytest.mark.parametrize("io,fmt", [("f16", FMT_F16), ("bf16", FMT_BF16)])
@pytest.mark.parametrize("diff", [False, True])
def test_method_mode_matches_brute(io, fmt, diff):
    L, D, w = 11, 8, 3
    q, k, q2, k2, v = (_rand((1, 1, L, D), s, io) for s in range(50, 55))
    c32, s32 = P.rope_table_f32(L, D)
    scale = 1 / np.sqrt(D)
    kw = dict(lam=0.8, q2=q2, k2=k2) if diff else {}
    got = A.attn_method(q, k, v, c32, s32, io, scale, window=w, **kw)[0, 0]
    bkw = dict(lam=0.8, q2=q2[0, 0].tolist(), k2=k2[0, 0].tolist()) if diff else {}
    want = np.array(brute_attention(q[0, 0].tolist(), k[0, 0].tolist(), v[0, 0].tolist(), scale, w,
                                    method=(c32.astype(float).tolist(), s32.astype(float).tolist(), fmt),
                                    **bkw))
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


@pytest.mark.parametrize("pairing,rd", [("half", 8), ("half", 4), ("adjacent", 4)])
@pytest.mark.parametrize("diff", [False, True])
def test_method_mode_rope_options_match_brute(pairing, rd, diff):
    L, D, w = 10, 8, 2
    io, fmt = "bf16", FMT_BF16
    q, k, q2, k2, v = (_rand((1, 1, L, D), s, io) for s in range(60, 65))
    c32, s32 = P.rope_table_f32(L, rd)
    scale = 1 / np.sqrt(D)
    kw = dict(lam=0.8, q2=q2, k2=k2) if diff else {}
    got = A.attn_method(q, k, v, c32, s32, io, scale, window=w, pairing=pairing, rotary_dim=rd, **kw)[0, 0]
    bkw = dict(lam=0.8, q2=q2[0, 0].tolist(), k2=k2[0, 0].tolist()) if diff else {}
    want = np.array(brute_attention(q[0, 0].tolist(), k[0, 0].tolist(), v[0, 0].tolist(), scale, w,
                                    method=(c32.astype(float).tolist(), s32.astype(float).tolist(), fmt),
                                    pairing=pairing, rotary_dim=rd, **bkw))
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)
    # the rows entry point agrees with the full one
    rows = np.array([0, 3, 9])
    r = A.attn_method_rows(q, k, v, c32, s32, io, scale, 0, 0, rows, window=w, pairing=pairing, rotary_dim=rd,
                           **kw)
    np.testing.assert_allclose(r, got[rows], rtol=0, atol=1e-14)


def test_def_mode_rope_options_match_brute():
    L, D = 9, 8
    q, k, v = (_rand((1, 1, L, D), s) for s in (70, 71, 72))
    got = A.attn_def(q, k, v, 0.3, window=-1, pairing="half", rotary_dim=4)[0, 0]
    want = np.array(brute_attention(q[0, 0].tolist(), k[0, 0].tolist(), v[0, 0].tolist(), 0.3, -1,
                                    pairing="half", rotary_dim=4))
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def test_rows_of_p_sum_to_one():
    L, D = 300, 64
    for w in (-1, 0, 5, 100):
        q, k, v = (_rand((L, D), s) for s in (1, 2, 3))
        _, Pm = A.masked_attention(q, k, v, 0.125, window=w, return_p=True)
        assert np.max(np.abs(Pm.sum(axis=1) - 1)) < 1e-12
        assert np.all(Pm >= 0)
        if w >= 0:
            i, j = np.indices(Pm.shape)
            assert np.all(Pm[np.abs(i - j) > w] == 0)


def test_window_at_least_L_equals_full_bitwise():
    L, D = 130, 64
    q, k, v = (_rand((1, 2, L, D), s) for s in (4, 5, 6))
    full = A.attn_def(q, k, v, 0.125, window=-1)
    for w in (L - 1, L, L + 7, 10 * L):
        np.testing.assert_array_equal(A.attn_def(q, k, v, 0.125, window=w), full)


def test_lambda_zero_equals_plain_bitwise():
    L, D = 70, 64
    q, k, q2, k2, v = (_rand((1, 2, L, D), s, "bf16") for s in range(60, 65))
    c32, s32 = P.rope_table_f32(L, D)
    for w in (-1, 9):
        plain = A.attn_method(q, k, v, c32, s32, "bf16", 0.125, window=w)
        diff0 = A.attn_method(q, k, v, c32, s32, "bf16", 0.125, window=w, lam=0.0, q2=q2, k2=k2)
        np.testing.assert_array_equal(diff0, plain)


def test_identical_branches_give_one_minus_lambda():
    L, D = 40, 16
    q, k, v = (_rand((1, 1, L, D), s) for s in (7, 8, 9))
    plain = A.attn_def(q, k, v, 0.3, window=6)
    d = A.attn_def(q, k, v, 0.3, window=6, lam=0.8, q2=q, k2=k)
    np.testing.assert_allclose(d, 0.2 * plain, rtol=0, atol=1e-14)


def test_single_position_and_zero_window_return_v():
    D = 64
    q, k, v = (_rand((1, 3, 1, D), s) for s in (10, 11, 12))
    np.testing.assert_array_equal(A.attn_def(q, k, v, 0.125), v)
    L = 37
    q, k, v = (_rand((1, 1, L, D), s) for s in (13, 14, 15))
    np.testing.assert_array_equal(A.attn_def(q, k, v, 0.125, window=0), v)
    c32, s32 = P.rope_table_f32(L, D)
    np.testing.assert_array_equal(A.attn_method(q, k, v, c32, s32, "f16", 0.125, window=0), v)
    # differential with w = 0: (1 - lambda) v
    d = A.attn_def(q, k, v, 0.125, window=0, lam=0.8, q2=k, k2=q)
    np.testing.assert_allclose(d, 0.2 * v, rtol=0, atol=1e-15)


def test_zero_queries_give_window_mean_of_v():
    L, D, w = 50, 8, 4
    k, v = _rand((1, 1, L, D), 16), _rand((1, 1, L, D), 17)
    q = np.zeros_like(k)
    got = A.attn_def(q, k, v, 0.125, window=w)[0, 0]
    for i in range(L):
        lo, hi = max(0, i - w), min(L, i + w + 1)
        np.testing.assert_allclose(got[i], v[0, 0, lo:hi].mean(axis=0), rtol=0, atol=1e-14)
    full = A.attn_def(q, k, v, 0.125)[0, 0]
    np.testing.assert_allclose(full, np.broadcast_to(v[0, 0].mean(axis=0), full.shape), rtol=0, atol=1e-14)


def test_dominant_key_returns_its_value_row():
    L, D = 30, 4
    rng = np.random.default_rng(18)
    kr = rng.standard_normal((L, D)) * 0.1
    qr = np.zeros((L, D))
    qr[:, 0] = 1.0
    j = 17
    kr[j, 0] = 400.0  # logit lead >= 40 after scale 0.125
    v = rng.standard_normal((L, D))
    out = A.masked_attention(qr, kr, v, 0.125)
    np.testing.assert_allclose(out, np.broadcast_to(v[j], out.shape), rtol=0, atol=1e-15)


def test_window_is_a_half_width_block_span_matches_pages():
    """A block of BLOCK_N consecutive queries under half-width w needs BLOCK_N + 2w keys."""
    fact = FACTS["window_block_span"]
    bn, w = fact["block_n"], fact["window"]
    L, D = 256, 8
    q, k, v = (_rand((L, D), s) for s in (19, 20, 21))
    rows = np.arange(100, 100 + bn)
    _, Pm = A.masked_attention(q, k, v, 0.125, window=w, rows=rows, return_p=True)
    used = np.flatnonzero((Pm > 0).any(axis=0))
    assert used.size == fact["keys_needed"]
    assert used.size > fact["block_kv"]  # a 64-wide tile is not enough, as the page warns
    assert used[0] == rows[0] - w and used[-1] == rows[-1] + w


def test_banded_equals_full_masked_matrix():
    L, D, w = 700, 16, 37
    q, k, v = (_rand((L, D), s) for s in (22, 23, 24))
    got = A.masked_attention(q, k, v, 0.2, window=w)
    S = 0.2 * (q @ k.T)
    i, j = np.indices(S.shape)
    S[np.abs(i - j) > w] = -np.inf
    Pm = np.exp(S - S.max(axis=1, keepdims=True))
    Pm /= Pm.sum(axis=1, keepdims=True)
    np.testing.assert_allclose(got, Pm @ v, rtol=0, atol=1e-13)


def test_rows_mode_matches_full():
    L, D = 200, 64
    for io, diff, w in (("f16", False, -1), ("bf16", True, 30)):
        q = _rand((2, 1, 2, L, D), 25, io)
        k = _rand((2, 1, 2, L, D), 26, io)
        v = _rand((1, 2, L, D), 27, io)
        c32, s32 = P.rope_table_f32(L, D)
        if diff:
            full = A.attn_method(q[0], k[0], v, c32, s32, io, 0.125, window=w, lam=0.8, q2=q[1], k2=k[1])
            rows = np.array([0, 5, 199, 100, 31])
            got = A.attn_method_rows(q[0], k[0], v, c32, s32, io, 0.125, 0, 1, rows, window=w,
                                     lam=0.8, q2=q[1], k2=k[1])
        else:
            full = A.attn_method(q[0], k[0], v, c32, s32, io, 0.125, window=w)
            rows = np.array([3, 0, 199, 64])
            got = A.attn_method_rows(q[0], k[0], v, c32, s32, io, 0.125, 0, 1, rows, window=w)
        np.testing.assert_allclose(got, full[0, 1, rows], rtol=0, atol=1e-14)
