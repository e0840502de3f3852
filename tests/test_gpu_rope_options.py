"""GPU parity of the RoPE options (sa3attn_forward_general through the binding).

The pages do not pin which dims RoPE pairs; besides the default (adjacent pairs over
the whole head dim) the library takes the half-split pairing (x[i], x[i + R/2]) and a
partial rotary width R (dims >= R pass through). Each case runs the HIP path and the
oracle (oracle.attention.attn_method with the same options, and its own [L][R/2]
table) on the same seeded inputs and compares every output element. The cases cover
the long-span kernel (plain, differential, windowed), the narrow-window kernel and
the short-sequence path, contiguous and strided.
"""

import numpy as np
import pytest

import oracle
from rope_attention_core_amd import synth

import gpu_common as G

pytestmark = pytest.mark.gpu


def _run_oracle(cfg, inp, pairing, rd):
    q, k, v = G.widen(inp, cfg)
    c32, s32 = oracle.rope_table_f32(cfg.L, rd, cfg.base)
    kw = dict(pairing=pairing, rotary_dim=rd)
    if cfg.diff:
        return oracle.attn_method(q[0], k[0], v, c32, s32, cfg.io, cfg.scale, window=cfg.window, lam=cfg.lam,
                                  q2=q[1], k2=k[1], **kw)
    return oracle.attn_method(q, k, v, c32, s32, cfg.io, cfg.scale, window=cfg.window, **kw)


def _run_gpu(cfg, inp, pairing, rd, strided=False):
    torch = G.torch_mod()
    q, k, v = (G.to_device(inp[n], cfg.io) for n in ("q", "k", "v"))
    if strided:
        q, k, v = (t.transpose(-2, -3).contiguous().transpose(-2, -3) for t in (q, k, v))
    c, s = G.device_table(cfg.L, rd, cfg.base)
    G.note(f"  rope: {cfg.name} B{cfg.B} H{cfg.H} L{cfg.L} w={cfg.window} diff={cfg.diff} {pairing} R={rd} "
           f"strided={strided}")
    out = G.sa3.forward(q, k, v, c, s, window=cfg.window, lam=cfg.lam, scale=cfg.scale,
                        out_dtype=G.out_torch_dtype(cfg.out_dtype), differential=cfg.diff,
                        pairing=pairing, rotary_dim=rd)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64)


SHAPES = [
    ("dit_2min", dict(H=2, L=600)),                  # long-span, plain
    ("samel_swa", dict(H=2, L=700, window=-1)),      # long-span, differential
    ("samel_swa", dict(H=2, L=900, window=100)),     # long-span, differential, windowed
    ("samel_w17", dict(H=2, L=800)),                 # narrow window
    ("dit_short", dict(H=3, L=150)),                 # short sequence
]


@pytest.mark.parametrize("pairing,rd", [("half", 64), ("half", 32), ("adjacent", 32), ("half", 16),
                                        ("adjacent", 48)])
@pytest.mark.parametrize("name,kw", SHAPES)
def test_rope_options(name, kw, pairing, rd):
    cfg = synth.config(name, seed=9500 + rd, **kw)
    inp = synth.make_inputs(cfg)
    G.assert_parity(_run_gpu(cfg, inp, pairing, rd), _run_oracle(cfg, inp, pairing, rd),
                    what=f"{name} {kw} {pairing} R={rd}", out=cfg.out_dtype)


@pytest.mark.parametrize("name,kw", SHAPES[:2] + SHAPES[3:])
def test_rope_options_strided(name, kw):
    cfg = synth.config(name, seed=9600, **kw)
    inp = synth.make_inputs(cfg)
    G.assert_parity(_run_gpu(cfg, inp, "half", 32, strided=True), _run_oracle(cfg, inp, "half", 32),
                    what=f"{name} {kw} half R=32 strided", out=cfg.out_dtype)


def test_default_options_through_the_general_path_match_the_default_call():
    """adjacent / R = D via a strided view (the general instances) equals the
    contiguous default call (the specialised instances) bit for bit (without the
    pre-pass, which would send this small contiguous grid to the key-split kernel)."""
    torch = G.torch_mod()
    cfg = synth.config("dit_2min", H=2, L=500, seed=9700)
    inp = synth.make_inputs(cfg)
    a = G.run_gpu(cfg, inp, prep="never")
    b = _run_gpu(cfg, inp, "adjacent", 64, strided=True)
    np.testing.assert_array_equal(a, b)
