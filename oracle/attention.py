"""Masked softmax attention in fp64, plain and differential, def and method modes.

Test infrastructure only (see the package header).

The attention core is QK^T -> softmax -> P.V ("Fixes the medium DiT's FP16-mixed
ONNX ..." discussion, sections "The bug" and "The fix"), with the softmax accumulated
in FP32 inside the fused kernel (same discussion, "The bug"). Here everything after
the RoPE cast-back is fp64 and unrounded, so the oracle is the exact result that an
FP32-accumulating kernel approximates.

Sliding window: key j is masked for query i when |i - j| > w, w being a half-width
(TensorRT engines README, section "Building your own": the window reaches WINDOW keys
to either side of a query, and a block of queries needs its own rows plus twice
WINDOW keys). w < 0 means full attention. There is no causal mask on this path.

Differential attention: out = softmax(S1) V - lambda * softmax(S2) V with the same
mask on both branches and RoPE applied to Q1, K1, Q2, K2; the two branch results are
subtracted after accumulation, in FP32 (TensorRT engines README, section "How the
kernels differ"). No per-head norm or extra factor is applied (none is described as
part of the core).

Evaluation order is the definition's. Rows are computed in chunks because each
output row depends only on its own row of scores; for a window only the keys with
|i - j| <= w are gathered, which leaves every softmax unchanged because masked keys
contribute exp(-inf) = 0. The row maximum is subtracted before exponentiation, the
standard identity softmax(s) = softmax(s - c).

Parity: pinned in tests/test_oracle_attention.py by the pure-Python brute force
(math.exp, math.fsum) on L <= 12, by the invariants (rows of P sum to 1; a window
>= L equals full attention; lambda = 0 equals plain attention; Q2 = Q1 and K2 = K1
gives (1 - lambda) times plain) and by closed forms (L = 1 and w = 0 give V; Q = 0
gives the window mean of V; one dominant key returns its V row).
"""

import numpy as np

from .rope import rotate_def, rotate_method, rope_angles

__all__ = ["softmax_rows", "masked_attention", "attn_def", "attn_method", "attn_method_rows"]

_CHUNK = 512


def softmax_rows(S):
    """Row softmax of an fp64 score matrix in which -inf marks masked entries."""
    S = np.asarray(S, dtype=np.float64)
    mx = S.max(axis=-1, keepdims=True)
    E = np.exp(S - mx)
    return E / E.sum(axis=-1, keepdims=True)


def masked_attention(qr, kr, v, scale, window=-1, rows=None, return_p=False):
    """softmax(scale * qr kr^T + M) v for one (batch, head).

    qr, kr, v: [L, D] fp64 (qr already rotated, as are kr). ``rows`` selects query
    rows (default: all). Returns out [len(rows), D]; with return_p also the full
    probability matrix [len(rows), L].
    """
    qr = np.asarray(qr, dtype=np.float64)
    kr = np.asarray(kr, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    L = kr.shape[0]
    rows = np.arange(qr.shape[0]) if rows is None else np.asarray(rows, dtype=np.int64)
    out = np.empty((rows.shape[0], v.shape[1]), dtype=np.float64)
    P_full = np.zeros((rows.shape[0], L), dtype=np.float64) if return_p else None
    for c0 in range(0, rows.shape[0], _CHUNK):
        rc = rows[c0:c0 + _CHUNK]
        if window >= 0:
            lo = max(0, int(rc.min()) - window)
            hi = min(L, int(rc.max()) + window + 1)
        else:
            lo, hi = 0, L
        keys = np.arange(lo, hi)
        S = scale * (qr[rc] @ kr[lo:hi].T)
        if window >= 0:
            S = np.where(np.abs(rc[:, None] - keys[None, :]) > window, -np.inf, S)
        P = softmax_rows(S)
        out[c0:c0 + _CHUNK] = P @ v[lo:hi]
        if return_p:
            P_full[c0:c0 + _CHUNK, lo:hi] = P
    if return_p:
        return out, P_full
    return out


def _core(qr, kr, v, scale, window, lam, q2r, k2r):
    B, H, L, D = v.shape
    out = np.empty((B, H, L, D), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            o = masked_attention(qr[b, h], kr[b, h], v[b, h], scale, window)
            if q2r is not None:
                o = o - lam * masked_attention(q2r[b, h], k2r[b, h], v[b, h], scale, window)
            out[b, h] = o
    return out


def _rope_kw(pairing, rotary_dim):
    # the default (adjacent, full width) is passed as no keywords at all
    kw = {}
    if pairing != "adjacent":
        kw["pairing"] = pairing
    if rotary_dim is not None:
        kw["rotary_dim"] = rotary_dim
    return kw


def attn_def(q, k, v, scale, window=-1, lam=0.0, q2=None, k2=None, base=10000.0,
             pairing="adjacent", rotary_dim=None):
    """def mode: RoPE in exact fp64 math (fp64 cos/sin), then fp64 attention.

    q, k, v, q2, k2: [B, H, L, D] fp64 values. Differential when q2/k2 are given.
    pairing / rotary_dim: the RoPE options of oracle.rope (default adjacent, full).
    """
    v = np.asarray(v, dtype=np.float64)
    L, D = v.shape[-2], v.shape[-1]
    R = D if rotary_dim is None else rotary_dim
    phi = rope_angles(L, R, base)
    c, s = np.cos(phi), np.sin(phi)
    kw = _rope_kw(pairing, rotary_dim)
    qr, kr = rotate_def(q, c, s, **kw), rotate_def(k, c, s, **kw)
    q2r = rotate_def(q2, c, s, **kw) if q2 is not None else None
    k2r = rotate_def(k2, c, s, **kw) if k2 is not None else None
    return _core(qr, kr, v, scale, window, lam, q2r, k2r)


def attn_method(q, k, v, cos32, sin32, io, scale, window=-1, lam=0.0, q2=None, k2=None,
                pairing="adjacent", rotary_dim=None):
    """method mode: FP32 RoPE with the FP32 table, RNE cast to ``io``, fp64 after.

    q, k, v, q2, k2: [B, H, L, D] fp64 values exactly representable in ``io``.
    cos32, sin32: the FP32 table [>=L, R/2] (R = rotary_dim, default D). Differential
    when q2/k2 are given.
    """
    v = np.asarray(v, dtype=np.float64)
    kw = _rope_kw(pairing, rotary_dim)
    qr = rotate_method(q, cos32, sin32, io, **kw)
    kr = rotate_method(k, cos32, sin32, io, **kw)
    q2r = rotate_method(q2, cos32, sin32, io, **kw) if q2 is not None else None
    k2r = rotate_method(k2, cos32, sin32, io, **kw) if k2 is not None else None
    return _core(qr, kr, v, scale, window, lam, q2r, k2r)


def attn_method_rows(q, k, v, cos32, sin32, io, scale, b, h, rows,
                     window=-1, lam=0.0, q2=None, k2=None, pairing="adjacent", rotary_dim=None):
    """method mode for selected query rows of one (b, h); returns [len(rows), D].

    Only the selected Q rows are rotated; all keys of the head are. Used to check
    sampled outputs of full-size runs one row at a time.
    """
    kw = _rope_kw(pairing, rotary_dim)
    rows = np.asarray(rows, dtype=np.int64)
    L = v.shape[-2]
    c = np.asarray(cos32, dtype=np.float32)[:L]
    s = np.asarray(sin32, dtype=np.float32)[:L]

    def rot_rows(x):
        # rotate only the requested rows: the table row follows the position
        return rotate_method_rows(np.asarray(x[b, h], dtype=np.float64)[rows], c[rows], s[rows], io, **kw)

    vh = np.asarray(v[b, h], dtype=np.float64)
    qr = np.zeros((L, v.shape[-1]))
    qr[rows] = rot_rows(q)
    kr = rotate_method(np.asarray(k[b, h], dtype=np.float64), c, s, io, **kw)
    out = masked_attention(qr, kr, vh, scale, window, rows=rows)
    if q2 is not None:
        q2r = np.zeros_like(qr)
        q2r[rows] = rot_rows(q2)
        k2r = rotate_method(np.asarray(k2[b, h], dtype=np.float64), c, s, io, **kw)
        out = out - lam * masked_attention(q2r, k2r, vh, scale, window, rows=rows)
    return out


def rotate_method_rows(x_rows, c_rows, s_rows, io, **kw):
    """rotate_method for rows whose table rows are given alongside (one per row)."""
    # rotate_method slices the table by the row count; passing per-row table rows
    # as a table of the same length keeps position m paired with its own cos/sin.
    return rotate_method(x_rows, c_rows, s_rows, io, **kw)
