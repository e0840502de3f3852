"""C-ABI checks that need no GPU: exports, status strings, validation, host table.

Validation runs before the library touches the device, so every error path below is
exercised with placeholder (never dereferenced) pointers. A call that passes
validation on a machine without a GPU must report SA3_ERR_DEVICE, not crash.
"""

import ctypes
import os
import re

import numpy as np
import pytest

import rope_attention_core_amd as sa3
from oracle import rope as P

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sa3attn.h")

SA3_OK, SA3_ERR_NULL, SA3_ERR_SHAPE, SA3_ERR_UNSUPPORTED, SA3_ERR_ARG, SA3_ERR_DEVICE = 0, -1, -2, -3, -4, -5
SA3_ERR_SCRATCH = -7


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sa3attn_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return sa3.load_library()


def test_library_exports_every_declared_function(lib):
    names = _declared_functions()
    assert len(names) >= 6
    for n in names:
        assert hasattr(lib, n), f"{n} declared in sa3attn.h but not exported"
    assert set(names) == set(sa3.EXPORTS)


def test_status_strings_and_version(lib):
    assert sa3.status_string(0) == "SA3_OK"
    for code in range(-7, 0):
        s = sa3.status_string(code)
        assert s.startswith("SA3_ERR_"), s
    assert "unknown" in sa3.status_string(12345)
    assert sa3.version() == (0, 6)


@pytest.mark.parametrize("L,D", [(1, 2), (37, 8), (8192, 16), (8192, 64), (8192, 128)])
def test_rope_table_matches_oracle_table(L, D):
    """The library's host table and the oracle's own table agree bit for bit.

    Both define theta_i as the fp64 value nearest base^(-2i/D) and round
    cos/sin(fp64(m) * theta_i) once to fp32; the two are computed independently.
    """
    c, s = sa3.rope_table(L, D)
    c0, s0 = P.rope_table_f32(L, D)
    np.testing.assert_array_equal(c.numpy(), c0)
    np.testing.assert_array_equal(s.numpy(), s0)


def test_rope_table_argument_errors(lib):
    buf = (ctypes.c_float * 64)()
    assert lib.sa3attn_rope_table(None, buf, 4, 8, 1e4) == SA3_ERR_NULL
    assert lib.sa3attn_rope_table(buf, buf, 0, 8, 1e4) == SA3_ERR_SHAPE
    assert lib.sa3attn_rope_table(buf, buf, 4, 7, 1e4) == SA3_ERR_SHAPE
    assert lib.sa3attn_rope_table(buf, buf, 4, 8, -1.0) == SA3_ERR_ARG
    assert lib.sa3attn_rope_table(buf, buf, 4, 8, float("nan")) == SA3_ERR_ARG


# Placeholder addresses, far apart so that no range overlaps unless a test wants it.
def _fake(i):
    return ctypes.c_void_p((i + 1) << 40)


def _desc(**kw):
    d = dict(q=_fake(1), k=_fake(2), v=_fake(3), cos=_fake(4), sin=_fake(5), out=_fake(6),
             B=1, H=2, L=64, D=64, window=-1, lambda_=0.0, scale=0.125, dtype=0, out_dtype=0,
             differential=0, stream=None)
    d.update(kw)
    return sa3._Desc(**d)


def _call(lib, **kw):
    return lib.sa3attn_forward_ex(ctypes.byref(_desc(**kw)))


@pytest.mark.parametrize("field", ["q", "k", "v", "cos", "sin", "out"])
def test_null_pointers_rejected(lib, field):
    assert _call(lib, **{field: ctypes.c_void_p(0)}) == SA3_ERR_NULL


def test_null_descriptor_rejected(lib):
    assert lib.sa3attn_forward_ex(None) == SA3_ERR_NULL


@pytest.mark.parametrize("kw,code", [
    (dict(B=0), SA3_ERR_SHAPE), (dict(H=-1), SA3_ERR_SHAPE), (dict(L=0), SA3_ERR_SHAPE),
    (dict(D=0), SA3_ERR_SHAPE), (dict(D=63), SA3_ERR_SHAPE), (dict(L=(1 << 24) + 1), SA3_ERR_SHAPE),
    (dict(B=1 << 20, H=1 << 12), SA3_ERR_SHAPE),
    (dict(D=32), SA3_ERR_UNSUPPORTED), (dict(D=96), SA3_ERR_UNSUPPORTED), (dict(D=256), SA3_ERR_UNSUPPORTED),
    (dict(D=128, L=(1 << 23) + 8), SA3_ERR_SHAPE),
    (dict(dtype=2), SA3_ERR_UNSUPPORTED), (dict(dtype=7), SA3_ERR_UNSUPPORTED),
    (dict(out_dtype=3), SA3_ERR_UNSUPPORTED),
    (dict(scale=float("nan")), SA3_ERR_ARG), (dict(scale=float("inf")), SA3_ERR_ARG),
    (dict(lambda_=float("nan")), SA3_ERR_ARG), (dict(differential=2), SA3_ERR_ARG),
    (dict(scale=3e38), SA3_ERR_ARG),
])
def test_bad_arguments_rejected(lib, kw, code):
    assert _call(lib, **kw) == code


def test_argument_swap_is_caught(lib):
    """Distinct prime sizes: a caller that swaps B/H/L/D lands on an unsupported D."""
    assert _call(lib, B=3, H=5, L=64, D=7) == SA3_ERR_SHAPE
    assert _call(lib, B=64, H=5, L=7, D=3) == SA3_ERR_SHAPE
    assert _call(lib, B=3, H=64, L=5, D=7) == SA3_ERR_SHAPE


@pytest.mark.parametrize("alias", ["q", "k", "v", "cos", "sin"])
def test_out_overlapping_an_input_rejected(lib, alias):
    base = _fake(9).value
    kw = {alias: ctypes.c_void_p(base), "out": ctypes.c_void_p(base + 64)}
    assert _call(lib, **kw) == SA3_ERR_ARG


def test_out_overlapping_second_branch_rejected(lib):
    # differential q spans two branches: out placed inside branch 2 must be caught
    base = _fake(9).value
    branch = 1 * 2 * 64 * 64 * 2
    assert _call(lib, differential=1, q=ctypes.c_void_p(base),
                 out=ctypes.c_void_p(base + branch + 128)) == SA3_ERR_ARG


def _gpu_present():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


# Calls below pass validation; with a GPU present they would launch on placeholder
# pointers, so they only run where there is none.
@pytest.mark.skipif(_gpu_present(), reason="placeholder pointers must never reach a real GPU")
def test_valid_call_without_gpu_reports_device_error(lib):
    assert _call(lib) == SA3_ERR_DEVICE
    assert _call(lib, B=3, H=5, L=7, D=64) == SA3_ERR_DEVICE
    # plain q spans one branch only: out just past it is no overlap
    base = _fake(9).value
    assert _call(lib, differential=0, q=ctypes.c_void_p(base),
                 out=ctypes.c_void_p(base + 2 * 64 * 64 * 2 + 128)) == SA3_ERR_DEVICE
    f = lib.sa3attn_forward
    assert f(_fake(1), _fake(2), _fake(3), _fake(4), _fake(5), _fake(6), 1, 2, 64, 64, -1, 0.0, 0.125,
             None) == SA3_ERR_DEVICE
    assert lib.sa3attn_forward_bf16(_fake(1), _fake(2), _fake(3), _fake(4), _fake(5), _fake(6), 1, 2, 64, 64,
                                    -1, 0.0, 0.125, None) == SA3_ERR_DEVICE
    # head dim 128, and the largest L it allows
    assert _call(lib, D=128) == SA3_ERR_DEVICE
    assert _call(lib, B=1, H=1, D=128, L=1 << 23) == SA3_ERR_DEVICE
    assert _call(lib, B=1, H=1, D=64, L=1 << 24) == SA3_ERR_DEVICE
    # rotary widths up to D: 80 is too wide for D = 64 but fits D = 128
    assert _call_general(lib, rope=_rope(1, 80), D=128) == SA3_ERR_DEVICE


def test_short_forms_validate_like_ex(lib):
    f = lib.sa3attn_forward
    assert f(None, _fake(2), _fake(3), _fake(4), _fake(5), _fake(6), 1, 2, 64, 64, -1, 0.0, 0.125, None) == SA3_ERR_NULL
    assert f(_fake(1), _fake(2), _fake(3), _fake(4), _fake(5), _fake(6), 1, 2, 64, 32, -1, 0.0, 0.125, None) == SA3_ERR_UNSUPPORTED
    assert f(_fake(1), _fake(2), _fake(3), _fake(4), _fake(5), _fake(6), 1, 2, 64, 64, -1, float("inf"), 0.125, None) == SA3_ERR_ARG


# ---- strided views (sa3attn_forward_strided) -----------------------------------------

def _strides(B=1, H=2, L=64, layout="bhld", **kw):
    """Element strides of a [B][H][L][64] view: "bhld" contiguous, "blhd" the
    [B][L][H][64] buffer a fused projection writes."""
    c = (H * L * 64, L * 64, 64) if layout == "bhld" else (L * H * 64, 64, H * 64)
    st = sa3._Strides()
    for f in ("q", "k", "v", "out"):
        getattr(st, f)[:] = kw.get(f, c)
    st.q_branch = kw.get("q_branch", B * H * L * 64)
    st.k_branch = kw.get("k_branch", B * H * L * 64)
    return st


def _call_strided(lib, st, **kw):
    return lib.sa3attn_forward_strided(ctypes.byref(_desc(**kw)), ctypes.byref(st))


def test_strided_null_strides_rejected(lib):
    assert lib.sa3attn_forward_strided(ctypes.byref(_desc()), None) == SA3_ERR_NULL
    assert lib.sa3attn_forward_strided(None, ctypes.byref(_strides())) == SA3_ERR_NULL


@pytest.mark.parametrize("field,val", [
    ("q", (2 * 64 * 64, 64 * 64, 60)),        # position stride shorter than a row
    ("k", (2 * 64 * 64, 64 * 64 + 4, 64)),    # not a multiple of 8 elements
    ("v", (-64, 64 * 64, 64)),                # negative
    ("out", (2 * 64 * 64, 64 * 64, 36)),
    ("q", (0, 0, 1 << 26)),                   # 32-bit row offsets would overflow
])
def test_strided_bad_strides_rejected(lib, field, val):
    assert _call_strided(lib, _strides(**{field: val})) == SA3_ERR_ARG


def test_strided_output_rows_must_be_distinct(lib):
    # H = 2 heads written to the same rows
    assert _call_strided(lib, _strides(out=(64 * 64, 0, 64))) == SA3_ERR_ARG
    # positions of one head interleaved with the other's: rows 64 apart, heads 64 apart
    assert _call_strided(lib, _strides(out=(2 * 64 * 64, 64, 64))) == SA3_ERR_ARG


def test_strided_out_overlapping_an_input_rejected(lib):
    # [B][L][H][64] q of 2 heads x 64 positions spans 2*64*64 elements; out starts inside
    base = _fake(9).value
    st = _strides(layout="blhd")
    assert _call_strided(lib, st, q=ctypes.c_void_p(base), out=ctypes.c_void_p(base + 64 * 64 * 2)) == SA3_ERR_ARG


def test_misaligned_pointer_rejected(lib):
    assert _call(lib, q=ctypes.c_void_p(_fake(1).value + 8)) == SA3_ERR_ARG
    assert _call(lib, out=ctypes.c_void_p(_fake(6).value + 2)) == SA3_ERR_ARG
    assert _call(lib, cos=ctypes.c_void_p(_fake(4).value + 4)) == SA3_ERR_ARG


def test_strided_differential_branch_stride_checked(lib):
    assert _call_strided(lib, _strides(q_branch=12), differential=1) == SA3_ERR_ARG
    assert _call_strided(lib, _strides(k_branch=-64), differential=1) == SA3_ERR_ARG


@pytest.mark.skipif(_gpu_present(), reason="placeholder pointers must never reach a real GPU")
def test_valid_strided_call_without_gpu_reports_device_error(lib):
    assert _call_strided(lib, _strides()) == SA3_ERR_DEVICE
    assert _call_strided(lib, _strides(layout="blhd")) == SA3_ERR_DEVICE
    assert _call_strided(lib, _strides(layout="blhd"), differential=1) == SA3_ERR_DEVICE
    # inputs may alias one another (they are only read): q, k, v in one buffer
    base = _fake(9).value
    assert _call_strided(lib, _strides(layout="blhd"), q=ctypes.c_void_p(base), k=ctypes.c_void_p(base),
                         v=ctypes.c_void_p(base)) == SA3_ERR_DEVICE


# ---- RoPE options (sa3attn_forward_general) ------------------------------------------

def _rope(pairing=0, rotary_dim=64):
    return sa3._Rope(pairing, rotary_dim)


def _call_general(lib, st=None, rope=None, **kw):
    return lib.sa3attn_forward_general(ctypes.byref(_desc(**kw)), ctypes.byref(st) if st is not None else None,
                                       ctypes.byref(rope) if rope is not None else None)


@pytest.mark.parametrize("pairing,rd", [(2, 64), (-1, 64), (0, 0), (0, 8), (1, 24), (1, 80), (0, 65), (1, -16)])
def test_bad_rope_options_rejected(lib, pairing, rd):
    assert _call_general(lib, rope=_rope(pairing, rd)) == SA3_ERR_ARG


def test_general_form_validates_like_ex(lib):
    assert lib.sa3attn_forward_general(None, None, None) == SA3_ERR_NULL
    assert _call_general(lib, rope=_rope(1, 32), q=ctypes.c_void_p(0)) == SA3_ERR_NULL
    assert _call_general(lib, rope=_rope(1, 32), D=96) == SA3_ERR_UNSUPPORTED
    assert _call_general(lib, st=_strides(q=(0, 0, 60)), rope=_rope(1, 32)) == SA3_ERR_ARG


def test_partial_rotary_table_extent_in_overlap_check(lib):
    # a [L][R/2] table of R = 32 is L * 16 floats: out right after it is no overlap,
    # out inside it is
    base = _fake(9).value
    tab = 64 * 16 * 4
    assert _call_general(lib, rope=_rope(0, 32), cos=ctypes.c_void_p(base),
                         out=ctypes.c_void_p(base + tab - 16)) == SA3_ERR_ARG


@pytest.mark.skipif(_gpu_present(), reason="placeholder pointers must never reach a real GPU")
def test_valid_general_calls_without_gpu_report_device_error(lib):
    assert _call_general(lib) == SA3_ERR_DEVICE
    for pairing in (0, 1):
        for rd in (16, 32, 48, 64):
            assert _call_general(lib, rope=_rope(pairing, rd)) == SA3_ERR_DEVICE
            assert _call_general(lib, st=_strides(layout="blhd"), rope=_rope(pairing, rd), differential=1) == \
                SA3_ERR_DEVICE
    base = _fake(9).value
    assert _call_general(lib, rope=_rope(0, 32), cos=ctypes.c_void_p(base),
                         out=ctypes.c_void_p(base + 64 * 16 * 4)) == SA3_ERR_DEVICE


# ---- workspace / pre-pass (sa3attn_workspace_bytes, sa3attn_forward_ws) -------------

AUTO, ALWAYS, NEVER, ONLY, REUSE = 0, 1, 2, 3, 4


def _ws_bytes(lib, policy=AUTO, **kw):
    n = ctypes.c_ulonglong(12345)
    rc = lib.sa3attn_workspace_bytes(ctypes.byref(_desc(**kw)), policy, ctypes.byref(n))
    return rc, n.value


def _lp(L):
    return (L + 63) // 64 * 64


def _tail_bytes(B, H, L, D=64, differential=0, window=-1, n_cu=256):
    """The split tail's share of the workspace, by the rule the header states: a grid of
    one 8-wave workgroup per query tile (256 rows, 128 differential; not the persistent
    grids of contiguous calls with more tiles than CUs and key spans <= 32 tiles, not
    the small plain D = 64 grids) whose last round holds r <= CUs / 2 tiles splits them
    in k = min(4, CUs // r) key ranges of >= 4 key tiles: r x k x 8 waves x 64 lanes x
    (D / 32 x 16 + 4) floats, then r counters in 256-byte units."""
    bm = 128 if differential else 256
    items = (L + bm - 1) // bm * B * H
    n_tiles = (L + 63) // 64
    span = n_tiles if window < 0 or window >= L - 1 else min(n_tiles, (2 * window + bm + 63) // 64 + 1)
    if items > n_cu and span <= 32:
        return 0                                   # persistent grid
    if D == 64 and not differential and (L + 255) // 256 * B * H < n_cu and (L + 63) // 64 * B * H <= 2 * n_cu:
        return 0                                   # small grid
    r = items % n_cu
    if r == 0 or 2 * r > n_cu:
        return 0
    k = min(4, n_cu // r)
    while k > 1 and span < 4 * k:
        k -= 1
    if k < 2:
        return 0
    return r * k * 8 * 64 * (D // 32 * 16 + 4) * 4 + (r * 4 + 255) // 256 * 256


@pytest.mark.parametrize("kw,policy,want", [
    # AUTO (256 compute units assumed without a device): key tiles visited by >= 10
    # query tiles of 256 rows (plain) / 18 of 128 (differential), >= 12 / 9 on persistent
    # grids, >= 3 at D = 128; small grids and split tails always
    (dict(B=2, H=24, L=4096), AUTO, 2 * 2 * 24 * 4096 * 64 * 2),
    (dict(B=1, H=24, L=2816), AUTO, 2 * 24 * _lp(2816) * 64 * 2),        # 11 visits, but 264 WGs: split tail
    (dict(B=1, H=20, L=2816), AUTO, 2 * 20 * _lp(2816) * 64 * 2),        # 11 visits, 220 WGs (one round)
    (dict(B=1, H=24, L=2304), AUTO, 0),                                  # 9 visits, 216 WGs
    (dict(B=1, H=24, L=2817), AUTO, 2 * 24 * _lp(2817) * 64 * 2),        # 12 visits, 288 WGs
    # plain D = 64 grids of fewer 256-row workgroups than compute units run 64-row tiles
    # with the pre-pass
    (dict(B=1, H=16, L=3072), AUTO, 2 * 16 * 3072 * 64 * 2),             # 768 of 64 rows: 256-row tiles, 12 visits
    (dict(B=1, H=24, L=1292), AUTO, 2 * 24 * _lp(1292) * 64 * 2),        # 144
    (dict(B=1, H=1, L=257), AUTO, 2 * 1 * _lp(257) * 64 * 2),            # 2
    (dict(B=1, H=12, L=2560), AUTO, 2 * 12 * 2560 * 64 * 2),             # 120 (480 of 64 rows)
    (dict(B=1, H=24, L=2560), AUTO, 2 * 24 * 2560 * 64 * 2),             # 240 (960 of 64 rows): 10 visits
    (dict(B=1, H=24, L=1344), AUTO, 2 * 24 * 1344 * 64 * 2),             # 144 (504 of 64 rows)
    (dict(B=1, H=24, L=1345), AUTO, 0),                                  # 144 (528 of 64 rows)
    (dict(B=1, H=24, L=2560, D=128), AUTO, 2 * 24 * 2560 * 128 * 2),     # D = 128: from 3 visits
    (dict(B=1, H=24, L=384, D=128), AUTO, 0),                            # D = 128, 2 visits
    (dict(B=1, H=32, L=1024, differential=1), AUTO, 0),                  # 8 visits
    (dict(B=1, H=32, L=1025, differential=1), AUTO, 3 * 32 * _lp(1025) * 64 * 2),   # 9, 288 WGs
    (dict(B=1, H=16, L=2048, differential=1), AUTO, 0),                  # 16 visits, one round
    (dict(B=1, H=8, L=4608, differential=1), AUTO, 3 * 8 * _lp(4608) * 64 * 2),   # 36 visits, 288 WGs: tail
    (dict(B=1, H=8, L=4096, window=1024, differential=1), AUTO, 3 * 8 * 4096 * 64 * 2),   # 18 visits, one round
    (dict(B=1, H=16, L=2049, differential=1), AUTO, 3 * 16 * _lp(2049) * 64 * 2),   # 17, 272 WGs
    # D = 128: the same 256 / 128 rows per query tile
    (dict(B=1, H=24, L=2816, D=128), AUTO, 2 * 24 * _lp(2816) * 128 * 2),   # split tail
    (dict(B=1, H=20, L=2816, D=128), AUTO, 2 * 20 * _lp(2816) * 128 * 2),
    (dict(B=1, H=24, L=2817, D=128), AUTO, 2 * 24 * _lp(2817) * 128 * 2),
    (dict(B=1, H=32, L=1024, D=128, differential=1), AUTO, 3 * 32 * 1024 * 128 * 2),
    (dict(B=1, H=32, L=1025, D=128, differential=1), AUTO, 3 * 32 * _lp(1025) * 128 * 2),
    # windows: a key tile of a half-width-w window is visited by about (2w + 64) / rows + 1
    # query tiles: 6 at w = 256, 8 at w = 384, 9 at w = 448 (128 rows); 10 at w = 1024,
    # 12 at w = 1280 (256 rows)
    (dict(B=1, H=16, L=8192, window=256, differential=1), AUTO, 0),
    (dict(B=1, H=16, L=8192, window=384, differential=1), AUTO, 0),
    (dict(B=1, H=16, L=8192, window=448, differential=1), AUTO, 3 * 16 * 8192 * 64 * 2),
    (dict(B=1, H=16, L=8192, window=1024), AUTO, 2 * 16 * 8192 * 64 * 2),   # 10 visits, tiles span 37 key tiles
    (dict(B=1, H=16, L=8192, window=768), AUTO, 0),                      # persistent, 8 visits
    (dict(B=1, H=16, L=8192, window=1280), AUTO, 2 * 16 * 8192 * 64 * 2),
    (dict(B=1, H=16, L=8192, window=256, differential=1), ALWAYS, 3 * 16 * 8192 * 64 * 2),
    (dict(B=1, H=16, L=8192, window=1024, differential=1), AUTO, 3 * 16 * 8192 * 64 * 2),
    # the single-span kernel (w <= 32, or L <= 256 at D = 64) has no pre-pass
    (dict(B=1, H=16, L=8192, window=17, differential=1), ALWAYS, 0),
    (dict(B=1, H=2, L=256), ALWAYS, 0),
    (dict(B=1, H=2, L=256, D=128), ALWAYS, 2 * 2 * 256 * 128 * 2),
    (dict(B=1, H=2, L=300), ALWAYS, 2 * 2 * _lp(300) * 64 * 2),
    (dict(B=2, H=24, L=4096), NEVER, 0),
    (dict(B=1, H=2, L=300), ONLY, 2 * 2 * _lp(300) * 64 * 2),
    (dict(B=1, H=2, L=300), REUSE, 2 * 2 * _lp(300) * 64 * 2),
    (dict(B=1, H=2, L=200), ONLY, 0),
])
def test_workspace_bytes(lib, kw, policy, want):
    if want:
        want += _tail_bytes(**kw)
    assert _ws_bytes(lib, policy, **kw) == (SA3_OK, want)
    B, H, L, D = kw["B"], kw["H"], kw["L"], kw.get("D", 64)
    prep = {AUTO: "auto", ALWAYS: "always", NEVER: "never", ONLY: "only", REUSE: "reuse"}[policy]
    assert sa3.workspace_bytes(B, H, L, D, window=kw.get("window", -1), differential=bool(kw.get("differential")),
                               prep=prep) == want


def test_workspace_bytes_errors(lib):
    n = ctypes.c_ulonglong(0)
    assert lib.sa3attn_workspace_bytes(None, AUTO, ctypes.byref(n)) == SA3_ERR_NULL
    assert lib.sa3attn_workspace_bytes(ctypes.byref(_desc()), AUTO, None) == SA3_ERR_NULL
    assert _ws_bytes(lib, 5)[0] == SA3_ERR_ARG
    assert _ws_bytes(lib, -1)[0] == SA3_ERR_ARG
    assert _ws_bytes(lib, D=96)[0] == SA3_ERR_UNSUPPORTED
    assert _ws_bytes(lib, L=0)[0] == SA3_ERR_SHAPE
    # pointers are not read: a shape-only descriptor is enough
    assert _ws_bytes(lib, ALWAYS, q=ctypes.c_void_p(0), out=ctypes.c_void_p(0), L=1000) == \
        (SA3_OK, 2 * 2 * _lp(1000) * 64 * 2)


def _call_ws(lib, ws, nbytes, policy=ALWAYS, st=None, rope=None, **kw):
    kw.setdefault("L", 1000)
    return lib.sa3attn_forward_ws(ctypes.byref(_desc(**kw)), ctypes.byref(st) if st is not None else None,
                                  ctypes.byref(rope) if rope is not None else None, ws, nbytes, policy)


def test_forward_ws_validation(lib):
    need = 2 * 2 * _lp(1000) * 64 * 2
    ws = _fake(20)
    assert lib.sa3attn_forward_ws(None, None, None, ws, need, ALWAYS) == SA3_ERR_NULL
    assert _call_ws(lib, None, need) == SA3_ERR_NULL
    assert _call_ws(lib, ws, need - 16) == SA3_ERR_ARG
    assert _call_ws(lib, ctypes.c_void_p(ws.value + 8), need) == SA3_ERR_ARG
    assert _call_ws(lib, ws, need, policy=5) == SA3_ERR_ARG
    for policy in (ONLY, REUSE):
        assert _call_ws(lib, None, need, policy=policy) == SA3_ERR_NULL
        assert _call_ws(lib, ws, need - 16, policy=policy) == SA3_ERR_ARG
    # the workspace overlaps an input or out
    for name in ("q", "k", "v", "cos", "sin", "out"):
        assert _call_ws(lib, ws, need, **{name: ctypes.c_void_p(ws.value + need - 64)}) == SA3_ERR_ARG, name
    # the usual checks still run first
    assert _call_ws(lib, ws, need, D=96) == SA3_ERR_UNSUPPORTED
    assert _call_ws(lib, ws, need, scale=float("nan")) == SA3_ERR_ARG
    assert _call_ws(lib, ws, need, rope=_rope(1, 80)) == SA3_ERR_ARG


@pytest.mark.skipif(_gpu_present(), reason="placeholder pointers must never reach a real GPU")
def test_valid_ws_calls_without_gpu_report_device_error(lib):
    need = 2 * 2 * _lp(1000) * 64 * 2
    ws = _fake(20)
    assert _call_ws(lib, ws, need) == SA3_ERR_DEVICE
    assert _call_ws(lib, ws, need + 4096) == SA3_ERR_DEVICE
    # no workspace needed: NEVER, AUTO below the threshold, the single-span kernel
    assert _call_ws(lib, None, 0, policy=NEVER) == SA3_ERR_DEVICE
    assert _call_ws(lib, None, 0, policy=AUTO, differential=1) == SA3_ERR_NULL   # split tail: the pre-pass runs
    assert _call_ws(lib, None, 0, policy=AUTO, differential=1, window=100) == SA3_ERR_DEVICE
    assert _call_ws(lib, None, 0, policy=AUTO) == SA3_ERR_NULL      # a small grid: the pre-pass runs
    assert _call_ws(lib, None, 0, policy=ALWAYS, window=17) == SA3_ERR_DEVICE
    assert _call_ws(lib, None, 0, policy=ALWAYS, L=200) == SA3_ERR_DEVICE
    assert _call_ws(lib, ws, need, policy=ONLY) == SA3_ERR_DEVICE
    assert _call_ws(lib, ws, need, policy=REUSE) == SA3_ERR_DEVICE
    assert _call_ws(lib, None, 0, policy=ONLY, window=17) == SA3_ERR_DEVICE
    # the workspace right after out is no overlap
    assert _call_ws(lib, ws, need, out=ctypes.c_void_p(ws.value - 2 * 1000 * 64 * 2)) == SA3_ERR_DEVICE
    assert _call_ws(lib, ws, 3 * 2 * _lp(1000) * 64 * 2 + _tail_bytes(1, 2, 1000, differential=1), differential=1,
                    st=_strides(layout="blhd"),
                    rope=_rope(1, 32)) == SA3_ERR_DEVICE


# ---- sa3attn_forward_noalloc: the static scratch as the pre-pass workspace -----------

SCRATCH = 64 << 20


def _call_na(lib, policy=ALWAYS, st=None, rope=None, **kw):
    return lib.sa3attn_forward_noalloc(ctypes.byref(_desc(**kw)), ctypes.byref(st) if st is not None else None,
                                       ctypes.byref(rope) if rope is not None else None, policy)


def test_noalloc_scratch_size_matches_header():
    text = open(HEADER).read()
    assert re.search(r"#define SA3ATTN_SCRATCH_BYTES \(64ull << 20\)", text)
    assert sa3.SCRATCH_BYTES == SCRATCH


def test_noalloc_validation(lib):
    assert lib.sa3attn_forward_noalloc(None, None, None, ALWAYS) == SA3_ERR_NULL
    assert _call_na(lib, policy=5) == SA3_ERR_ARG
    assert _call_na(lib, D=96) == SA3_ERR_UNSUPPORTED
    assert _call_na(lib, q=None) == SA3_ERR_NULL
    assert _call_na(lib, scale=float("inf")) == SA3_ERR_ARG
    assert _call_na(lib, rope=_rope(1, 80)) == SA3_ERR_ARG
    # a pre-pass workspace beyond the scratch: the medium DiT's differential shape
    # (3 x 2 x 24 x 4096 x 64 x 2 bytes = 72 MiB) under the policies that insist on it
    big = dict(B=2, H=24, L=4096, differential=1, dtype=1, out_dtype=2)
    rc, need = _ws_bytes(lib, ALWAYS, **big)
    assert rc == SA3_OK and need > SCRATCH
    for policy in (ALWAYS, ONLY, REUSE):
        assert _call_na(lib, policy=policy, **big) == SA3_ERR_SCRATCH


@pytest.mark.skipif(_gpu_present(), reason="placeholder pointers must never reach a real GPU")
def test_valid_noalloc_calls_without_gpu_report_device_error(lib):
    # within the scratch (the long latent's plain shape: 48 MiB), and AUTO beyond it
    # (which then runs without the pre-pass)
    long = dict(B=2, H=24, L=4096, dtype=1, out_dtype=2)
    rc, need = _ws_bytes(lib, ALWAYS, **long)
    assert rc == SA3_OK and 0 < need <= SCRATCH
    for policy in (AUTO, ALWAYS, NEVER, ONLY, REUSE):
        assert _call_na(lib, policy=policy, **long) == SA3_ERR_DEVICE
    assert _call_na(lib, policy=AUTO, B=2, H=24, L=4096, differential=1, dtype=1, out_dtype=2) == SA3_ERR_DEVICE
    assert _call_na(lib, policy=ALWAYS, window=17, L=5000) == SA3_ERR_DEVICE
