"""GPU: bf16 V beyond fp16's range, on every kernel path, against the oracle.

P.V runs on fp16 operands for bf16 inputs as well, and a bf16 |v| >= 65536 has no fp16
value. The kernels detect the non-finite accumulators this leaves, look up the largest
finite |v| of the keys the workgroup visited and redo the work with V scaled by an exact
power of two. These tests scale 1% of the V rows of every head by 2^17 (|v| up to about
5e5) and, in some heads, put a few values of +-3e38 (near bf16's largest finite value;
1e38 on differential calls, whose FP32 subtraction would otherwise overflow where the
fp64 oracle does not). The error bar scales with the largest |v| of the head
(2e-3 x max|v|, the arithmetic's relative accuracy), next to the usual row cosine on
plain calls. On differential calls the row cosine is not a measure of accuracy here:
where both branches weigh the same large V rows, out = O1 - lambda O2 cancels to a
small row while the error stays relative to the large values (about 3e-5 max|v|, the
fp16 rounding of P), so only the max-abs bar applies to them.
Heads without large values must come out bitwise as in a call where no head has any.
"""

import numpy as np
import pytest

from rope_attention_core_amd import synth

import gpu_common as G

pytestmark = pytest.mark.gpu


def bf16_bits(x64):
    return synth.to_storage(x64, "bf16")


def widen_bf16(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def big_v(cfg, seed, huge=3.0e38, huge_heads=(0,)):
    """cfg's inputs with 1% of V rows per head x 2^17 and, in `huge_heads`, a few
    elements of +-huge."""
    inp = synth.make_inputs(cfg)
    v = widen_bf16(inp["v"])
    rng = np.random.default_rng(seed)
    n = max(1, int(round(0.01 * cfg.L)))
    for b in range(cfg.B):
        for h in range(cfg.H):
            rows = rng.choice(cfg.L, size=n, replace=False)
            v[b, h, rows, :] *= 2.0 ** 17
            if h in huge_heads:
                for _ in range(3):
                    i, d = int(rng.integers(0, cfg.L)), int(rng.integers(0, cfg.D))
                    v[b, h, i, d] = huge if rng.integers(0, 2) else -huge
    out = dict(inp)
    out["v"] = bf16_bits(v)
    return out


def check(cfg, inp, got, rows=None, what=""):
    vmax = np.abs(widen_bf16(inp["v"])).max(axis=(2, 3))          # [B, H]
    for b in range(cfg.B):
        for h in range(cfg.H):
            if rows is None:
                want = G.run_oracle(cfg.with_(B=1, H=1), {
                    "q": inp["q"][..., b:b + 1, h:h + 1, :, :], "k": inp["k"][..., b:b + 1, h:h + 1, :, :],
                    "v": inp["v"][b:b + 1, h:h + 1]})[0, 0]
                g = got[b, h]
            else:
                want = G.run_oracle_rows(cfg, inp, b, h, rows)
                g = got[b, h, rows]
            G.assert_parity(g, want, atol=2e-3 * vmax[b, h], min_cos=-1.0 if cfg.diff else G.MIN_ROW_COS,
                            what=f"{what} b{b} h{h} max|v| {vmax[b, h]:.3g}")


CASES = [
    # (name, overrides, forward kwargs, huge value)
    ("long-span fused", dict(L=1292, H=2), dict(prep="never"), 3.0e38),
    ("key-split pre-pass", dict(L=1292, H=2), dict(prep="always"), 3.0e38),
    ("long-span 2-wave pre-pass windowed", dict(L=1292, H=2, window=300), dict(prep="always"), 3.0e38),
    ("long-span pre-pass", dict(L=2000, H=24), dict(prep="always"), 3.0e38),
    ("long-span D128", dict(L=700, H=2, D=128), dict(prep="never"), 3.0e38),
    ("long-span D128 pre-pass", dict(L=700, H=2, D=128), dict(prep="always"), 3.0e38),
    ("long-span windowed diff", dict(L=1500, H=2, window=100, lam=0.8, diff=True), dict(prep="never"), 1.0e38),
    ("single-span w17 diff", dict(L=1000, H=2, window=17, lam=0.8, diff=True), {}, 1.0e38),
    ("single-span w17 plain", dict(L=1000, H=2, window=17), {}, 3.0e38),
    ("single-span L200", dict(L=200, H=3), {}, 3.0e38),
    ("single-span L256 diff", dict(L=256, H=2, lam=0.8, diff=True), {}, 1.0e38),
    ("single-span L50", dict(L=50, H=2), {}, 3.0e38),
]


@pytest.mark.parametrize("name,over,kw,huge", CASES, ids=[c[0].replace(" ", "-") for c in CASES])
def test_vrange_paths(name, over, kw, huge):
    base = "samel_swa" if over.get("diff") else "dit_long"
    over = dict(over, B=1, seed=40 + len(name), spike_frac=0.0, out="f32")
    cfg = synth.config(base, **over)
    inp = big_v(cfg, 500 + len(name), huge=huge)
    got = G.run_gpu(cfg, inp, **kw)
    assert np.all(np.isfinite(got)), f"{name}: non-finite output"
    rows = None
    if cfg.H > 4:  # many heads: the edges of the 256-row tiles and random rows of each
        rng = np.random.default_rng(7)
        rows = np.unique(np.concatenate([np.arange(0, cfg.L, 256), np.arange(255, cfg.L, 256), [cfg.L - 1],
                                         rng.integers(0, cfg.L, 16)]))
    check(cfg, inp, got, rows=rows, what=name)


@pytest.mark.parametrize("prep", ["never", "always"])
def test_vrange_persistent_window_sampled(prep):
    """The persistent grid whose key-tile pipeline runs on into the next query tile
    (differential, w = 256, 384 query tiles): a redone tile restarts the next one cold."""
    cfg = synth.config("samel_swa", B=1, H=12, L=4096, seed=71)
    inp = big_v(cfg, 72, huge=1.0e38, huge_heads=(0, 5))
    got = G.run_gpu(cfg, inp, prep=prep)
    assert np.all(np.isfinite(got))
    rows = np.unique(np.concatenate([np.arange(0, 140), np.arange(3950, 4096), np.arange(1000, 1300)]))
    vmax = np.abs(widen_bf16(inp["v"])).max(axis=(2, 3))
    for h in (0, 1, 5, 11):
        want = G.run_oracle_rows(cfg, inp, 0, h, rows)
        G.assert_parity(got[0, h, rows], want, atol=2e-3 * vmax[0, h], min_cos=-1.0, what=f"persistent h{h}")


@pytest.mark.parametrize("prep", ["never", "always"])
def test_vrange_other_heads_bitwise(prep):
    """Only the workgroups that met a large V redo their work: heads without one come
    out bitwise as in a call whose V has no large values at all."""
    cfg = synth.config("dit_long", B=1, H=3, L=1100, seed=81, spike_frac=0.0, out="f32")
    inp = synth.make_inputs(cfg)
    v = widen_bf16(inp["v"])
    v[0, 1, 17, 5] = 1.0e6
    v[0, 1, 900, 0] = -3.0e38
    big = dict(inp, v=bf16_bits(v))
    a = G.run_gpu(cfg, inp, prep=prep)
    b = G.run_gpu(cfg, big, prep=prep)
    assert np.array_equal(a[0, 0], b[0, 0]) and np.array_equal(a[0, 2], b[0, 2])
    assert not np.array_equal(a[0, 1], b[0, 1])
    vmax = np.abs(v[0, 1]).max()
    G.assert_parity(b[0, 1], G.run_oracle(cfg, big)[0, 1], atol=2e-3 * vmax, what="the head with large values")
