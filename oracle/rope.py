"""Rotary position embedding (RoPE): frequencies, the FP32 table, rotations.

Test infrastructure only (see the package header).

What the pages fix and what this module reads into them:

* RoPE runs in FP32 and is cast back to the activation dtype before QK^T
  ("Fixes the medium DiT's FP16-mixed ONNX ..." discussion, section "The bug").
* The cos/sin values come from a table computed on the host in FP32 and frozen
  ahead of time, with no trig in the graph (sa3_trt README, section "DiT
  precision", fp8 tier). The table is sized to a maximum length.
* A bf16 angle at about 4155 rad has a spacing of 32 rad, more than 2*pi, which
  destroys position information; this is why RoPE must stay FP32 (sa3_trt README,
  section "DiT precision", the retired bf16 tier; TensorRT engines README,
  section "Other things worth knowing").

Readings where the pages are silent (each listed in the design notes):

* pairs are adjacent, (x[2i], x[2i+1]), over the full head dim (the pages do not
  pin the pairing; the half-split pairing (x[i], x[i + R/2]) and a partial rotary
  width R < D, with the trailing D - R dims passed through, are provided as
  options, see ``pairing`` and ``rotary_dim`` below);
* theta_i = base ** (-2 i / D), i = 0 .. D/2-1, base 10000, as the fp64 value
  nearest the real number;
* positions are m = 0 .. L-1 with no offset;
* the FP32 table is one rounding of the fp64 value cos(fp64(m) * theta_i);
* the FP32 rotation is r0 = fl(fl(x0 c) - fl(x1 s)), r1 = fl(fl(x0 s) + fl(x1 c)),
  each product and sum rounded to FP32 separately (no fused multiply-add);
* the cast back to the IO dtype rounds to nearest-even.

Options of rotate_def / rotate_f32 / rotate_method: ``pairing`` "adjacent" (default)
or "half"; ``rotary_dim`` R (default: the whole head dim), even, R <= D; the table
then has R/2 columns (theta_i = base ** (-2 i / R)) and dims R.. D-1 are returned
unchanged. Pinned in tests/test_oracle_rope.py: the half-split rotation equals the
adjacent one on permuted dims, bit for bit; a partial rotation equals the full
rotation of the first R dims (with D := R) and the identity elsewhere; both against
the exact-rational brute force; and the relative-position invariant for half-split.

Parity: rope_frequencies, rope_table_f32, rotate_def and rotate_method are pinned in
tests/test_oracle_rope.py by closed forms (theta_0 = 1, theta_31 = 10^-3.875 at D=64,
m = 0 is the identity, D = 2 rotates by m rad), by invariants (each pair's norm is
preserved; <R_m q, R_n k> depends only on n - m), by the pure-Python brute force
(math.cos / exact Fraction rounding), and by the bf16-angle negative control.
"""

import decimal

import numpy as np

from .rounding import f32, round_io, f32_to_bf16_bits, bf16_bits_to_f64

__all__ = [
    "rope_frequencies",
    "rope_angles",
    "rope_table_f32",
    "rope_table_bf16_angle",
    "rotate_def",
    "rotate_f32",
    "rotate_method",
    "PAIRINGS",
]


def rope_frequencies(D, base=10000.0):
    """theta_i = base ** (-2 i / D) for i = 0 .. D/2 - 1: the fp64 value nearest the real one.

    Evaluated with 50-digit decimal arithmetic and rounded once to fp64, so the value
    does not depend on which libm pow() is at hand (two common ones differ in the last
    bit for some i, which moves fp32 table entries at large positions).
    """
    if D < 2 or D % 2:
        raise ValueError("D must be even and >= 2")
    with decimal.localcontext() as ctx:
        ctx.prec = 50
        b = decimal.Decimal(float(base))
        return np.array([float(b ** (decimal.Decimal(-2 * i) / decimal.Decimal(D))) for i in range(D // 2)],
                        dtype=np.float64)


def rope_angles(L, D, base=10000.0):
    """phi[m, i] = m * theta_i for m = 0 .. L-1, fp64, shape [L, D/2]."""
    m = np.arange(L, dtype=np.float64)
    return m[:, None] * rope_frequencies(D, base)[None, :]


def rope_table_f32(L, D, base=10000.0):
    """The host FP32 cos/sin table: fp32(cos(phi)), fp32(sin(phi)), each [L, D/2].

    One rounding from the fp64 value (sa3_trt README, section "DiT precision":
    position cos/sin computed host-side and frozen as a constant).
    """
    phi = rope_angles(L, D, base)
    return f32(np.cos(phi)), f32(np.sin(phi))


def rope_table_bf16_angle(L, D, base=10000.0):
    """Negative control: the table a bf16-evaluated angle produces.

    Position, frequency and their product are each rounded to bf16 before the
    trig, as a weakly typed bf16 graph would do (sa3_trt README, section "DiT
    precision", retired bf16 tier). Returned as fp32 cos/sin plus the bf16 angle.
    """
    def bf(x):
        return bf16_bits_to_f64(f32_to_bf16_bits(f32(x)))

    m = bf(np.arange(L, dtype=np.float64))
    th = bf(rope_frequencies(D, base))
    phi = bf(m[:, None] * th[None, :])
    return f32(np.cos(phi)), f32(np.sin(phi)), phi


PAIRINGS = ("adjacent", "half")


def _split(x, pairing, rotary_dim):
    """The two members of each rotated pair and the pass-through tail, along the last axis."""
    D = x.shape[-1]
    R = D if rotary_dim is None else int(rotary_dim)
    if R < 2 or R % 2 or R > D:
        raise ValueError("rotary_dim must be even, >= 2 and <= D")
    if pairing == "adjacent":
        x0, x1 = x[..., 0:R:2], x[..., 1:R:2]
    elif pairing == "half":
        x0, x1 = x[..., :R // 2], x[..., R // 2:R]
    else:
        raise ValueError(f"pairing must be one of {PAIRINGS}")
    return x0, x1, x[..., R:]


def _merge(r0, r1, tail, pairing):
    """Inverse of _split: put the rotated pair members back and append the tail."""
    n = r0.shape[-1]
    out = np.empty(r0.shape[:-1] + (2 * n + tail.shape[-1],), dtype=r0.dtype)
    if pairing == "adjacent":
        out[..., 0:2 * n:2] = r0
        out[..., 1:2 * n:2] = r1
    else:
        out[..., :n] = r0
        out[..., n:2 * n] = r1
    out[..., 2 * n:] = tail
    return out


def rotate_def(x, cos, sin, pairing="adjacent", rotary_dim=None):
    """Exact-math rotation in fp64.

    x: [..., L, D] fp64; cos, sin: [>=L, R/2] (any float dtype, widened to fp64).
    For each pair (x0, x1) (adjacent: x[2i], x[2i+1]; half: x[i], x[i + R/2]) with the
    table column i: r0 = x0 c - x1 s ; r1 = x0 s + x1 c. Dims >= R are unchanged.
    """
    x = np.asarray(x, dtype=np.float64)
    L = x.shape[-2]
    c = np.asarray(cos, dtype=np.float64)[:L]
    s = np.asarray(sin, dtype=np.float64)[:L]
    x0, x1, tail = _split(x, pairing, rotary_dim)
    return _merge(x0 * c - x1 * s, x0 * s + x1 * c, tail, pairing)


def rotate_f32(x, cos32, sin32, pairing="adjacent", rotary_dim=None):
    """The method's FP32 rotation, before the cast back: returns float32 [..., L, D].

    x: [..., L, D] values exactly representable in FP32 (fp64 array); cos32, sin32:
    the FP32 table [>=L, R/2]. Every product and sum is an FP32 operation rounded on
    its own (numpy float32 ufuncs, no fusion):
    r0 = fl(fl(x0 c) - fl(x1 s)), r1 = fl(fl(x0 s) + fl(x1 c)). Dims >= R are copied.
    """
    x32 = np.asarray(x, dtype=np.float64).astype(np.float32)
    L = x32.shape[-2]
    c = np.asarray(cos32, dtype=np.float32)[:L]
    s = np.asarray(sin32, dtype=np.float32)[:L]
    x0, x1, tail = _split(x32, pairing, rotary_dim)
    a = np.multiply(x0, c, dtype=np.float32)
    b = np.multiply(x1, s, dtype=np.float32)
    r0 = np.subtract(a, b, dtype=np.float32)
    a = np.multiply(x0, s, dtype=np.float32)
    b = np.multiply(x1, c, dtype=np.float32)
    r1 = np.add(a, b, dtype=np.float32)
    return _merge(r0, r1, tail, pairing)


def rotate_method(x, cos32, sin32, io, pairing="adjacent", rotary_dim=None):
    """The method's rotation: FP32 arithmetic (rotate_f32), then RNE cast to ``io``.

    Returns the IO-dtype values widened to fp64 (the pass-through dims are IO values
    already, so the cast leaves them unchanged).
    """
    return round_io(rotate_f32(x, cos32, sin32, pairing, rotary_dim), io)
