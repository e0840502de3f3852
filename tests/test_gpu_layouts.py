"""GPU parity on strided views (sa3attn_forward_strided through the binding).

The fused projection of a DiT writes q, k, v as [B, L, H, D] (position-major); the
library reads such buffers in place through element strides instead of needing a
transpose to [B, H, L, D]. Every case is compared, element by element, with the
oracle on the same values in the contiguous [B, H, L, D] order, and with the
contiguous call of the library (which must give identical bits: the strides change
addresses only, never the arithmetic).
"""

import numpy as np
import pytest

from rope_attention_core_amd import synth

import gpu_common as G

pytestmark = pytest.mark.gpu


def _blhd_view(t):
    """A [.., B, H, L, D] tensor copied into a [.., B, L, H, D] buffer, returned as a
    [.., B, H, L, D] view of that buffer (non-contiguous, last dimension contiguous)."""
    return t.transpose(-2, -3).contiguous().transpose(-2, -3)


def _run(cfg, inp, q, k, v, out=None, **kw):
    torch = G.torch_mod()
    c, s = G.device_table(cfg.L, cfg.D, cfg.base)
    res = G.sa3.forward(q, k, v, c, s, window=cfg.window, lam=cfg.lam, scale=cfg.scale, out=out,
                        out_dtype=G.out_torch_dtype(cfg.out_dtype), differential=cfg.diff, **kw)
    torch.cuda.synchronize()
    return res


CASES = [
    # (config, overrides): long-span plain, long-span differential, narrow window,
    # short sequence
    ("dit_2min", dict(H=3, L=700)),
    ("samel_swa", dict(H=2, L=900, window=-1)),
    ("samel_swa", dict(H=2, L=1500, window=300)),
    ("samel_w17", dict(H=3, L=1000)),
    ("dit_2min", dict(H=3, L=1000, window=9, io="bf16", out="f32")),
    ("dit_short", dict(H=4, L=200)),
    ("samel_swa", dict(H=2, L=130, window=-1)),
]


@pytest.mark.parametrize("name,kw", CASES)
@pytest.mark.parametrize("strided_out", [False, True])
def test_blhd_inputs(name, kw, strided_out):
    torch = G.torch_mod()
    cfg = synth.config(name, seed=9100 + kw.get("L", 0), **kw)
    inp = synth.make_inputs(cfg)
    q, k, v = (G.to_device(inp[n], cfg.io) for n in ("q", "k", "v"))
    G.note(f"  strided: {cfg.name} {kw} out strided={strided_out}")
    qs, ks, vs = _blhd_view(q), _blhd_view(k), _blhd_view(v)
    assert not qs.is_contiguous() and qs.stride(-1) == 1
    # the fused path, and the pre-pass path for the differential cases (on small plain
    # full-attention grids the pre-pass would send the contiguous call to the key-split
    # kernel, which views never take)
    for prep in ("never", "always") if cfg.diff else ("never",):
        base = _run(cfg, inp, q, k, v, prep=prep)
        out = None
        if strided_out:
            B, H, L, D = v.shape
            out = torch.empty((B, L, H, D), dtype=G.out_torch_dtype(cfg.out_dtype), device="cuda").transpose(1, 2)
        got = _run(cfg, inp, qs, ks, vs, out=out, prep=prep)
        assert torch.equal(got.contiguous(), base), f"strided call differs from the contiguous one (prep {prep})"
        G.assert_parity(got.float().cpu().numpy().astype(np.float64), G.run_oracle(cfg, inp),
                        what=f"{name} {kw} blhd prep {prep}", out=cfg.out_dtype)


def test_heads_of_a_wider_buffer():
    """q, k, v as slices of one [B, L, 3H, D] buffer (a fused QKV projection)."""
    torch = G.torch_mod()
    cfg = synth.config("dit_2min", H=4, L=517, seed=9300)
    inp = synth.make_inputs(cfg)
    q, k, v = (G.to_device(inp[n], cfg.io) for n in ("q", "k", "v"))
    base = _run(cfg, inp, q, k, v, prep="never")
    B, H, L, D = v.shape
    qkv = torch.empty((B, L, 3 * H, D), dtype=q.dtype, device="cuda")
    qkv[:, :, 0:H] = q.transpose(1, 2)
    qkv[:, :, H:2 * H] = k.transpose(1, 2)
    qkv[:, :, 2 * H:] = v.transpose(1, 2)
    got = _run(cfg, inp, qkv[:, :, 0:H].transpose(1, 2), qkv[:, :, H:2 * H].transpose(1, 2),
               qkv[:, :, 2 * H:].transpose(1, 2))
    assert torch.equal(got, base)
