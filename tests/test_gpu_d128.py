"""GPU parity at head dim 128 (the long-span kernel's D = 128 instances).

Every case runs the HIP path and the oracle on the same seeded inputs and compares the
outputs element by element (sampled rows at the full long-latent size). The cases
cover plain and differential attention, full and windowed, a short sequence inside one
key tile, ragged lengths, both IO dtypes and output casts, strided [B, L, H, D] views
and the RoPE options (half-split pairing, partial rotary widths up to 128).
"""

import numpy as np
import pytest

import oracle
from rope_attention_core_amd import synth

import gpu_common as G

pytestmark = pytest.mark.gpu


def _d128(name, **kw):
    return synth.config(name, D=128, **kw)


CASES = [
    ("dit_2min", dict(H=3, L=700)),                                # plain, ragged
    ("dit_2min", dict(H=2, L=1000, io="bf16", out="f32")),          # plain bf16 -> f32
    ("dit_short", dict(H=4, L=40)),                                 # one partial key tile
    ("dit_2min", dict(H=2, L=1, out="f32")),                        # a single position
    ("samel_swa", dict(H=2, L=700, window=-1)),                     # differential, full
    ("samel_swa", dict(H=2, L=1500, window=200)),                   # differential, windowed
    ("samel_w17", dict(H=2, L=900)),                                # differential, w = 17
    ("dit_2min", dict(H=2, L=900, window=9, io="bf16", out="bf16")),  # plain, narrow window
    ("dit_2min", dict(H=2, L=513, window=0)),                       # diagonal only
]


@pytest.mark.parametrize("name,kw", CASES)
def test_d128_parity(name, kw):
    cfg = _d128(name, seed=9900 + kw["L"], **kw)
    inp = synth.make_inputs(cfg)
    G.assert_parity(G.run_gpu(cfg, inp), G.run_oracle(cfg, inp), what=f"D=128 {name} {kw}", out=cfg.out_dtype)


def test_d128_long_latent_sampled():
    """The long latent (B2 H12 L4096 D128, bf16, 1% spiked keys): sampled rows of
    every (b, h) against the oracle's row-wise evaluation."""
    cfg = synth.config("dit_long_d128")
    inp = synth.make_inputs(cfg)
    got = G.run_gpu(cfg, inp)
    rng = np.random.default_rng(11)
    for b in range(cfg.B):
        for h in range(cfg.H):
            rows = np.unique(np.concatenate([[0, cfg.L - 1], rng.integers(0, cfg.L, 6)]))
            want = G.run_oracle_rows(cfg, inp, b, h, rows)
            G.assert_parity(got[b, h, rows], want, what=f"dit_long_d128 b{b} h{h}", out=cfg.out_dtype)


def test_d128_strided_views_match_contiguous():
    torch = G.torch_mod()
    for name, kw in (("dit_2min", dict(H=3, L=600)), ("samel_swa", dict(H=2, L=800, window=100))):
        cfg = _d128(name, seed=9950, **kw)
        inp = synth.make_inputs(cfg)
        q, k, v = (G.to_device(inp[n], cfg.io) for n in ("q", "k", "v"))
        c, s = G.device_table(cfg.L, cfg.D, cfg.base)
        call = dict(window=cfg.window, lam=cfg.lam, scale=cfg.scale, out_dtype=G.out_torch_dtype(cfg.out_dtype),
                    differential=cfg.diff)
        base = G.sa3.forward(q, k, v, c, s, **call)
        qs, ks, vs = (t.transpose(-2, -3).contiguous().transpose(-2, -3) for t in (q, k, v))
        got = G.sa3.forward(qs, ks, vs, c, s, **call)
        torch.cuda.synchronize()
        assert torch.equal(got, base), f"{name}: strided call differs from the contiguous one"
        G.assert_parity(got.float().cpu().numpy().astype(np.float64), G.run_oracle(cfg, inp),
                        what=f"D=128 {name} strided", out=cfg.out_dtype)


def _oracle_opts(cfg, inp, pairing, rd):
    q, k, v = G.widen(inp, cfg)
    c32, s32 = oracle.rope_table_f32(cfg.L, rd, cfg.base)
    kw = dict(pairing=pairing, rotary_dim=rd)
    if cfg.diff:
        return oracle.attn_method(q[0], k[0], v, c32, s32, cfg.io, cfg.scale, window=cfg.window, lam=cfg.lam,
                                  q2=q[1], k2=k[1], **kw)
    return oracle.attn_method(q, k, v, c32, s32, cfg.io, cfg.scale, window=cfg.window, **kw)


@pytest.mark.parametrize("pairing,rd", [("half", 128), ("half", 64), ("adjacent", 96), ("half", 112),
                                        ("adjacent", 16)])
@pytest.mark.parametrize("name,kw", [("dit_2min", dict(H=2, L=600)), ("samel_swa", dict(H=2, L=700, window=50))])
def test_d128_rope_options(name, kw, pairing, rd):
    cfg = _d128(name, seed=9970 + rd, **kw)
    inp = synth.make_inputs(cfg)
    q, k, v = (G.to_device(inp[n], cfg.io) for n in ("q", "k", "v"))
    c, s = G.device_table(cfg.L, rd, cfg.base)
    G.note(f"  rope D=128: {name} {kw} {pairing} R={rd}")
    out = G.sa3.forward(q, k, v, c, s, window=cfg.window, lam=cfg.lam, scale=cfg.scale,
                        out_dtype=G.out_torch_dtype(cfg.out_dtype), differential=cfg.diff,
                        pairing=pairing, rotary_dim=rd)
    G.torch_mod().cuda.synchronize()
    G.assert_parity(out.float().cpu().numpy().astype(np.float64), _oracle_opts(cfg, inp, pairing, rd),
                    what=f"D=128 {name} {pairing} R={rd}", out=cfg.out_dtype)
