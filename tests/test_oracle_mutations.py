"""Plant plausible mistakes in the oracle (CPU only) and check that a pin catches each.

Every mutation below is applied with monkeypatch to the oracle's own functions; the
pins are the ordinary tests in test_oracle_*.py, called directly. A mutation that no
pin catches would mean the oracle could carry that mistake unnoticed.
"""

import numpy as np
import pytest

import oracle.attention as A
import oracle.rope as P
import oracle.rounding as R

import test_oracle_attention as TA
import test_oracle_rope as TP
import test_oracle_rounding as TR


def _interleave(r0, r1):
    out = np.empty(r0.shape[:-1] + (2 * r0.shape[-1],), dtype=r0.dtype)
    out[..., 0::2] = r0
    out[..., 1::2] = r1
    return out


def _fails(fn, *args):
    try:
        fn(*args)
    except AssertionError:
        return True
    return False


def _any_fails(checks):
    return any(_fails(*c) for c in checks)


# --- rope mutations --------------------------------------------------------------

def _rot_sign_flip(x, cos, sin, **kw):
    x = np.asarray(x, dtype=np.float64)
    L = x.shape[-2]
    c, s = np.asarray(cos, float)[:L], np.asarray(sin, float)[:L]
    x0, x1 = x[..., 0::2], x[..., 1::2]
    return _interleave(x0 * c + x1 * s, -x0 * s + x1 * c)


def _rot_half_split(x, cos, sin, **kw):
    # pairs (i, i + D/2) instead of adjacent pairs
    x = np.asarray(x, dtype=np.float64)
    L, D = x.shape[-2], x.shape[-1]
    c, s = np.asarray(cos, float)[:L], np.asarray(sin, float)[:L]
    x0, x1 = x[..., : D // 2], x[..., D // 2:]
    return np.concatenate([x0 * c - x1 * s, x0 * s + x1 * c], axis=-1)


def _freq_wrong(D, base=10000.0):
    i = np.arange(D // 2, dtype=np.float64)
    return np.power(np.float64(base), -1.0 * i / D)


def _rot_f32_fused(x, cos32, sin32, **kw):
    # rounds once at the end instead of after every FP32 operation
    x = np.asarray(x, dtype=np.float64)
    L = x.shape[-2]
    c = np.asarray(cos32, np.float64)[:L]
    s = np.asarray(sin32, np.float64)[:L]
    x0, x1 = x[..., 0::2], x[..., 1::2]
    return _interleave(x0 * c - x1 * s, x0 * s + x1 * c).astype(np.float32)


def _rot_f32_fma(x, cos32, sin32, **kw):
    # r0 = fma(x0, c, -fl(x1 s)): one product left unrounded
    x = np.asarray(x, dtype=np.float64)
    L = x.shape[-2]
    c = np.asarray(cos32, np.float32)[:L].astype(np.float64)
    s = np.asarray(sin32, np.float32)[:L].astype(np.float64)
    x0, x1 = x[..., 0::2], x[..., 1::2]
    b = (x1 * s).astype(np.float32).astype(np.float64)
    d = (x1 * c).astype(np.float32).astype(np.float64)
    return _interleave((x0 * c - b).astype(np.float32), (x0 * s + d).astype(np.float32))


def _rot_method_no_cast(x, cos32, sin32, io, **kw):
    x32 = np.asarray(x, dtype=np.float64).astype(np.float32)
    L = x32.shape[-2]
    c, s = np.asarray(cos32, np.float32)[:L], np.asarray(sin32, np.float32)[:L]
    x0, x1 = x32[..., 0::2], x32[..., 1::2]
    return _interleave(x0 * c - x1 * s, x0 * s + x1 * c).astype(np.float64)


ROPE_DEF_PINS = [
    (TP.test_d2_rotates_by_m_radians,),
    (TP.test_rotate_def_matches_brute,),
    (TP.test_dot_depends_only_on_offset,),
]


@pytest.mark.parametrize("mut", [_rot_sign_flip, _rot_half_split])
def test_rotation_mistakes_are_caught(monkeypatch, mut):
    monkeypatch.setattr(P, "rotate_def", mut)
    monkeypatch.setattr(A, "rotate_def", mut)
    assert _any_fails(ROPE_DEF_PINS + [(TA.test_def_mode_matches_brute, 5, 4, -1)])


def test_frequency_mistake_is_caught(monkeypatch):
    monkeypatch.setattr(P, "rope_frequencies", _freq_wrong)
    assert _fails(TP.test_theta_closed_forms)
    assert _fails(TP.test_table_is_one_rounding_of_fp64_trig)


@pytest.mark.parametrize("mut", [_rot_f32_fused, _rot_f32_fma])
def test_fp32_rotation_mistakes_are_caught(monkeypatch, mut):
    monkeypatch.setattr(P, "rotate_f32", mut)
    assert _fails(TP.test_rotate_f32_bit_exact_vs_rational)


@pytest.mark.parametrize("mut", [_rot_method_no_cast])
@pytest.mark.parametrize("io", ["f16", "bf16"])
def test_method_rotation_mistakes_are_caught(monkeypatch, mut, io):
    monkeypatch.setattr(P, "rotate_method", mut)
    monkeypatch.setattr(A, "rotate_method", mut)
    from oracle.brute import FMT_BF16, FMT_F16
    fmt = FMT_F16 if io == "f16" else FMT_BF16
    assert _any_fails([(TP.test_rotate_method_bit_exact_vs_rational, io, fmt, 64),
                       (TA.test_method_mode_matches_brute, io, fmt, False)])


# --- rounding mutations ----------------------------------------------------------

def _bf16_truncate(x32):
    x32 = np.ascontiguousarray(np.asarray(x32, dtype=np.float32))
    return (x32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def _bf16_ties_away(x32):
    x32 = np.ascontiguousarray(np.asarray(x32, dtype=np.float32))
    u = x32.view(np.uint32).astype(np.uint64)
    return ((u + np.uint64(0x8000)) >> np.uint64(16)).astype(np.uint16)


@pytest.mark.parametrize("mut", [_bf16_truncate, _bf16_ties_away])
def test_bf16_rounding_mistakes_are_caught(monkeypatch, mut):
    monkeypatch.setattr(R, "f32_to_bf16_bits", mut)
    assert _any_fails([(TR.test_bf16_matches_exact_rne_random,), (TR.test_bf16_ties_round_to_even,)])


# --- attention mutations ---------------------------------------------------------

_orig_masked = A.masked_attention


def _attn_transposed(qr, kr, v, scale, window=-1, rows=None, return_p=False):
    return _orig_masked(kr, qr, v, scale, window, rows, return_p)


def _attn_no_scale(qr, kr, v, scale, window=-1, rows=None, return_p=False):
    return _orig_masked(qr, kr, v, 1.0, window, rows, return_p)


def _attn_window_off_by_one(qr, kr, v, scale, window=-1, rows=None, return_p=False):
    return _orig_masked(qr, kr, v, scale, window + 1 if window >= 0 else window, rows, return_p)


def _attn_full_width_window(qr, kr, v, scale, window=-1, rows=None, return_p=False):
    return _orig_masked(qr, kr, v, scale, window // 2 if window >= 0 else window, rows, return_p)


ATTN_PINS = [
    (TA.test_def_mode_matches_brute, 8, 4, 2),
    (TA.test_def_mode_matches_brute, 12, 8, -1),
    (TA.test_window_is_a_half_width_block_span_matches_pages,),
    (TA.test_zero_queries_give_window_mean_of_v,),
    (TA.test_single_position_and_zero_window_return_v,),
]


@pytest.mark.parametrize("mut", [_attn_transposed, _attn_no_scale, _attn_window_off_by_one,
                                 _attn_full_width_window])
def test_attention_mistakes_are_caught(monkeypatch, mut):
    monkeypatch.setattr(A, "masked_attention", mut)
    assert _any_fails(ATTN_PINS)


def test_differential_sign_mistake_is_caught(monkeypatch):
    orig = A._core

    def plus_lambda(qr, kr, v, scale, window, lam, q2r, k2r):
        return orig(qr, kr, v, scale, window, -lam, q2r, k2r)

    monkeypatch.setattr(A, "_core", plus_lambda)
    assert _fails(TA.test_def_mode_differential_matches_brute, 0.8, 2)
    assert _fails(TA.test_identical_branches_give_one_minus_lambda)


def test_softmax_without_normalisation_is_caught(monkeypatch):
    def unnormalised(S):
        S = np.asarray(S, dtype=np.float64)
        return np.exp(S - S.max(axis=-1, keepdims=True))

    monkeypatch.setattr(A, "softmax_rows", unnormalised)
    assert _fails(TA.test_rows_of_p_sum_to_one)
    assert _fails(TA.test_def_mode_matches_brute, 8, 4, -1)


# --- RoPE option mutations -------------------------------------------------------

_rotate_f32 = P.rotate_f32


def _half_wrong_partner(x, cos32, sin32, pairing="adjacent", rotary_dim=None):
    # half-split pairs taken as (i, i + R/2 - 1): off by one in the partner index
    if pairing != "half":
        return _rotate_f32(x, cos32, sin32, pairing, rotary_dim)
    R = x.shape[-1] if rotary_dim is None else rotary_dim
    y = np.array(x, copy=True)
    y[..., R // 2:R] = np.roll(np.asarray(x)[..., R // 2:R], 1, axis=-1)
    return _rotate_f32(y, cos32, sin32, pairing, rotary_dim)


def _partial_rotates_tail(x, cos32, sin32, pairing="adjacent", rotary_dim=None):
    # the table is reused cyclically over the whole head dim instead of stopping at R
    R = x.shape[-1] if rotary_dim is None else rotary_dim
    if R == x.shape[-1]:
        return _rotate_f32(x, cos32, sin32, pairing, rotary_dim)
    c = np.concatenate([np.asarray(cos32)] * (x.shape[-1] // R), axis=-1)
    s = np.concatenate([np.asarray(sin32)] * (x.shape[-1] // R), axis=-1)
    return _rotate_f32(x, c, s, pairing)


@pytest.mark.parametrize("mut", [_half_wrong_partner, _partial_rotates_tail])
def test_rotation_option_mistakes_are_caught(monkeypatch, mut):
    monkeypatch.setattr(P, "rotate_f32", mut)
    checks = [(TP.test_half_split_is_adjacent_on_permuted_dims, 32),
              (TP.test_partial_rotary_leaves_the_tail_and_rotates_the_head, 32, "adjacent"),
              (TP.test_partial_rotary_leaves_the_tail_and_rotates_the_head, 32, "half")]
    from oracle.brute import FMT_F16
    checks += [(TP.test_rotation_options_bit_exact_vs_rational, r, p, D, "f16", FMT_F16)
               for r, p, D in ((32, "half", 64), (64, "half", 64), (32, "adjacent", 64), (96, "half", 128))]
    assert _any_fails(checks)
