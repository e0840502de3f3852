"""GPU checks of the 128-key steps of the long-span kernel (one round per query tile,
with the pre-pass).

Such grids walk the keys in pairs of 64-key tiles, with K and V^T in LDS rings; an item
of an odd number of key tiles ends with one tile past its range, masked as keys past the
item's end. Cases: odd and even tile counts, full attention and windows (the mask at
both window edges), plain and differential (the per-quarter fast path), fp16 and bf16,
head dim 128, [B, L, H, D] views (the general instances), fp16 output; every case
against the oracle on rows at query-tile edges, the last rows and random rows, plus
run-to-run bits.
"""

import numpy as np
import pytest

from rope_attention_core_amd import synth

import gpu_common as G

pytestmark = pytest.mark.gpu


def _kv_bytes(cfg):
    return (3 if cfg.diff else 2) * cfg.B * cfg.H * ((cfg.L + 63) // 64 * 64) * cfg.D * 2


CASES = [
    # name, overrides, strided: grids of at most one round of query tiles that no split
    # tail applies to (256 tiles; 248 differential), so every tile runs the pair steps
    ("dit_long", dict(B=1, H=16, L=4000), False),                       # 63 key tiles (odd)
    ("dit_long", dict(B=1, H=16, L=4096, io="f16", out="f16"), False),  # 64 (even), fp16
    ("dit_long", dict(B=1, H=16, L=4000, window=700), False),           # window edges, 23-24 tiles
    ("dit_long", dict(B=1, H=16, L=4000), True),                        # [B, L, H, D] views
    ("samel_swa", dict(B=1, H=8, L=3900, window=-1), False),            # differential, 61 tiles (odd)
    ("samel_swa", dict(B=1, H=8, L=3900, window=900), False),           # differential window
    ("dit_long_d128", dict(B=1, H=16, L=4000), False),                  # head dim 128, odd
]


def _rows(cfg, rng):
    bm = 128 if cfg.diff else 256
    edges = [0, 1, cfg.L - 2, cfg.L - 1] + [t * bm + d for t in (1, cfg.L // bm // 2, cfg.L // bm) for d in (-1, 0)]
    return np.unique(np.clip(np.concatenate([edges, rng.integers(0, cfg.L, 10)]), 0, cfg.L - 1))


@pytest.mark.parametrize("name,kw,strided", CASES)
def test_pair_steps_parity(name, kw, strided):
    torch = G.torch_mod()
    cfg = synth.config(name, seed=16000 + kw["L"] + (7 if strided else 0), **kw)
    nb = G.sa3.workspace_bytes(cfg.B, cfg.H, cfg.L, cfg.D, window=cfg.window, differential=cfg.diff, prep="always")
    assert nb == _kv_bytes(cfg), "a split tail would apply to this shape"
    inp = synth.make_inputs(cfg)
    q, k, v = (G.to_device(inp[n], cfg.io) for n in ("q", "k", "v"))
    if strided:
        q, k, v = (t.transpose(-2, -3).contiguous().transpose(-2, -3) for t in (q, k, v))
    c, s = G.device_table(cfg.L, cfg.D, cfg.base)
    G.note(f"  pair steps: {name} {kw} strided={strided}")
    call = dict(window=cfg.window, lam=cfg.lam, scale=cfg.scale, out_dtype=G.out_torch_dtype(cfg.out_dtype),
                differential=cfg.diff, prep="always")
    a = G.sa3.forward(q, k, v, c, s, **call)
    b = G.sa3.forward(q, k, v, c, s, **call)
    torch.cuda.synchronize()
    assert torch.equal(a, b), "two calls differ"
    got = a.float().cpu().numpy().astype(np.float64)
    assert np.isfinite(got).all()
    rng = np.random.default_rng(16100)
    for bh in (0, cfg.H // 2, cfg.H - 1):
        rows = _rows(cfg, rng)
        want = G.run_oracle_rows(cfg, inp, 0, bh, rows)
        G.assert_parity(got[0, bh, rows], want, what=f"{name} {kw} h{bh}", out=cfg.out_dtype)
