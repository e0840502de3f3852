"""Pure-Python brute force for tiny inputs: the pin for the numpy oracle.

Test infrastructure only (see the package header).

Written independently of rope.py / attention.py / rounding.py: nested Python lists,
math.cos / math.sin / math.exp, math.fsum for every sum, and exact rational
arithmetic (fractions.Fraction) with a hand-written round-to-nearest-even for the
FP32 rotation and the casts. Nothing here imports numpy.

It restates the same definition (RoPE on adjacent pairs, theta_i = base^(-2i/D),
positions 0..L-1, scores scaled then masked for |i-j| > w, softmax, P.V, and the
differential difference) so that a dropped term, wrong sign, wrong index or
transposed operand in the vectorised oracle shows up as a mismatch.
"""

import math
from fractions import Fraction

__all__ = [
    "FMT_F32", "FMT_F16", "FMT_BF16",
    "round_fraction", "round_float",
    "brute_theta", "brute_rotate_def", "brute_rotate_method", "brute_attention",
]

# (significand bits including the implicit one, minimum normal exponent, maximum exponent)
FMT_F32 = (24, -126, 127)
FMT_F16 = (11, -14, 15)
FMT_BF16 = (8, -126, 127)


def _floor_log2(a):
    """floor(log2(a)) for a positive Fraction, exactly."""
    n, d = a.numerator, a.denominator
    e = n.bit_length() - d.bit_length()
    # 2^e <= a < 2^(e+1) must hold; adjust by one if needed
    if e >= 0:
        if n < (d << e):
            e -= 1
    else:
        if (n << -e) < d:
            e -= 1
    return e


def round_fraction(x, fmt):
    """Round an exact rational to the nearest value of a binary format (RNE).

    Returns a Fraction, or a float infinity on overflow. Subnormals are handled
    by clamping the exponent at the minimum normal exponent.
    """
    p, emin, emax = fmt
    x = Fraction(x)
    if x == 0:
        return Fraction(0)
    sign = -1 if x < 0 else 1
    a = -x if x < 0 else x
    e = max(_floor_log2(a), emin)
    ulp = Fraction(2) ** (e - (p - 1))
    q = a / ulp
    n = q.numerator // q.denominator
    rem = q - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    r = n * ulp
    largest = (Fraction(2) - Fraction(2) ** (1 - p)) * Fraction(2) ** emax
    if r > largest:
        return sign * math.inf
    return sign * r


def round_float(x, fmt):
    """round_fraction for a Python float input, returned as a Python float."""
    if math.isnan(x):
        return x
    if math.isinf(x):
        return x
    r = round_fraction(Fraction(x), fmt)
    return float(r) if not isinstance(r, float) else r


def brute_theta(D, base):
    return [base ** (-2.0 * i / D) for i in range(D // 2)]


def _pair_index(i, R, pairing):
    """Dims of pair i: (2i, 2i+1) adjacent, (i, i + R/2) half-split."""
    return (2 * i, 2 * i + 1) if pairing == "adjacent" else (i, i + R // 2)


def brute_rotate_def(x, D, base, pairing="adjacent", rotary_dim=None):
    """x: list over positions of lists of D floats. Exact-math RoPE (fp64 trig) of the
    first R = rotary_dim (default D) dims, pairs chosen by ``pairing``; the rest copied."""
    R = D if rotary_dim is None else rotary_dim
    th = brute_theta(R, base)
    out = []
    for m, row in enumerate(x):
        r = list(row)
        for i in range(R // 2):
            phi = m * th[i]
            c, s = math.cos(phi), math.sin(phi)
            j0, j1 = _pair_index(i, R, pairing)
            a, b = row[j0], row[j1]
            r[j0] = math.fsum([a * c, -b * s])
            r[j1] = math.fsum([a * s, b * c])
        out.append(r)
    return out


def brute_rotate_method(x, cos32, sin32, io_fmt, pairing="adjacent", rotary_dim=None):
    """FP32 rotation with every product and sum rounded on its own, exact rationals.

    x: list over positions of lists of D floats (exact IO values); cos32, sin32:
    lists over positions of lists of R/2 floats holding FP32 table values.
    io_fmt=None returns the FP32 results without the cast back. Dims >= R are copied.
    """
    out = []
    for m, row in enumerate(x):
        D = len(row)
        R = D if rotary_dim is None else rotary_dim
        r = list(row)
        for i in range(R // 2):
            j0, j1 = _pair_index(i, R, pairing)
            c, s = Fraction(cos32[m][i]), Fraction(sin32[m][i])
            a, b = Fraction(row[j0]), Fraction(row[j1])
            ac = round_fraction(a * c, FMT_F32)
            bs = round_fraction(b * s, FMT_F32)
            as_ = round_fraction(a * s, FMT_F32)
            bc = round_fraction(b * c, FMT_F32)
            r0 = round_fraction(ac - bs, FMT_F32)
            r1 = round_fraction(as_ + bc, FMT_F32)
            if io_fmt is not None:
                r0, r1 = round_fraction(r0, io_fmt), round_fraction(r1, io_fmt)
            r[j0] = float(r0)
            r[j1] = float(r1)
        out.append(r)
    return out


def _attend(qr, kr, v, scale, window):
    L, D = len(kr), len(v[0])
    out = []
    for i in range(len(qr)):
        s = []
        for j in range(L):
            if window >= 0 and abs(i - j) > window:
                s.append(None)
            else:
                s.append(scale * math.fsum(qr[i][d] * kr[j][d] for d in range(D)))
        mx = max(x for x in s if x is not None)
        e = [0.0 if x is None else math.exp(x - mx) for x in s]
        tot = math.fsum(e)
        out.append([math.fsum(e[j] * v[j][d] for j in range(L)) / tot for d in range(D)])
    return out


def brute_attention(q, k, v, scale, window=-1, lam=0.0, q2=None, k2=None,
                    base=10000.0, method=None, pairing="adjacent", rotary_dim=None):
    """Attention for one head, lists [L][D]. Differential when q2/k2 are given.

    method=None rotates in exact math (def mode); method=(cos32, sin32, io_fmt)
    rotates with the FP32 emulation and casts to the IO format (method mode).
    pairing / rotary_dim as in the rotations.
    """
    D = len(q[0])

    def rot(x):
        if method is None:
            return brute_rotate_def(x, D, base, pairing, rotary_dim)
        cos32, sin32, io_fmt = method
        return brute_rotate_method(x, cos32, sin32, io_fmt, pairing, rotary_dim)

    o = _attend(rot(q), rot(k), v, scale, window)
    if q2 is not None:
        o2 = _attend(rot(q2), rot(k2), v, scale, window)
        o = [[o[i][d] - lam * o2[i][d] for d in range(D)] for i in range(len(o))]
    return o
