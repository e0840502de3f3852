"""Shared helpers of the GPU parity tests: run the HIP path and the oracle on one input.

The GPU side gets the library's own RoPE table (sa3attn_rope_table); the oracle builds
its own (oracle.rope.rope_table_f32). The two tables are checked equal on the CPU
(tests/test_abi.py); nothing here passes a GPU result to the oracle.
"""

import sys

import numpy as np

import oracle
import rope_attention_core_amd as sa3
from rope_attention_core_amd import synth

# Parity bar for FP16/BF16 inputs: max-abs error and per-row cosine against the oracle.
ATOL = 2e-3
MIN_ROW_COS = 0.99995


def note(msg):
    print(msg, file=sys.stderr, flush=True)


def torch_mod():
    import torch
    return torch


def to_device(arr, io):
    torch = torch_mod()
    if io == "f16":
        t = torch.from_numpy(np.ascontiguousarray(arr))
    else:
        t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16)
    return t.cuda()


def out_torch_dtype(name):
    torch = torch_mod()
    return {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}[name]


_tables = {}


def device_table(L, D=64, base=10000.0):
    key = (L, D, base)
    if key not in _tables:
        c, s = sa3.rope_table(L, D, base)
        _tables[key] = (c.cuda(), s.cuda())
    return _tables[key]


def run_gpu(cfg, inp, out=None, **kw):
    """Run the library on cfg's inputs; returns the output as an fp64 numpy array."""
    torch = torch_mod()
    q, k, v = (to_device(inp[n], cfg.io) for n in ("q", "k", "v"))
    c, s = device_table(cfg.L, cfg.D, cfg.base)
    note(f"  gpu: {cfg.name} B{cfg.B} H{cfg.H} L{cfg.L} {cfg.io} w={cfg.window} lam={cfg.lam} "
         f"diff={cfg.diff} out={cfg.out_dtype} seed={cfg.seed}")
    res = sa3.forward(q, k, v, c, s, window=cfg.window, lam=cfg.lam, scale=cfg.scale, out=out,
                      out_dtype=out_torch_dtype(cfg.out_dtype), differential=cfg.diff, **kw)
    torch.cuda.synchronize()
    return res.float().cpu().numpy().astype(np.float64)


def widen(inp, cfg):
    q = oracle.widen_io(inp["q"], cfg.io)
    k = oracle.widen_io(inp["k"], cfg.io)
    v = oracle.widen_io(inp["v"], cfg.io)
    return q, k, v


def run_oracle(cfg, inp):
    """Full method-mode oracle output [B, H, L, D]."""
    q, k, v = widen(inp, cfg)
    c32, s32 = oracle.rope_table_f32(cfg.L, cfg.D, cfg.base)
    if cfg.diff:
        return oracle.attn_method(q[0], k[0], v, c32, s32, cfg.io, cfg.scale, window=cfg.window,
                                  lam=cfg.lam, q2=q[1], k2=k[1])
    return oracle.attn_method(q, k, v, c32, s32, cfg.io, cfg.scale, window=cfg.window)


def run_oracle_rows(cfg, inp, b, h, rows):
    q, k, v = widen(inp, cfg)
    c32, s32 = oracle.rope_table_f32(cfg.L, cfg.D, cfg.base)
    if cfg.diff:
        return oracle.attn_method_rows(q[0], k[0], v, c32, s32, cfg.io, cfg.scale, b, h, rows,
                                       window=cfg.window, lam=cfg.lam, q2=q[1], k2=k[1])
    return oracle.attn_method_rows(q, k, v, c32, s32, cfg.io, cfg.scale, b, h, rows, window=cfg.window)


def row_cosines(got, want):
    g = got.reshape(-1, got.shape[-1])
    w = want.reshape(-1, want.shape[-1])
    num = (g * w).sum(axis=1)
    den = np.linalg.norm(g, axis=1) * np.linalg.norm(w, axis=1)
    cos = np.where(den > 0, num / np.where(den > 0, den, 1), 1.0)
    return cos


def half_ulp(want, out):
    """Half a unit in the last place of the output dtype at |want| (0 for fp32 output).

    The final cast to a 16-bit output is the method's own last rounding; for |out| >= 4
    fp16's half-ulp alone is 1.95e-3, so the arithmetic bar is applied on top of it.
    """
    a = np.abs(np.asarray(want, dtype=np.float64))
    if out == "f32":
        return np.zeros_like(a)
    bits = {"f16": 10, "bf16": 7}[out]
    emin = {"f16": -14, "bf16": -126}[out]
    e = np.floor(np.log2(np.maximum(a, 2.0 ** emin)))
    return 2.0 ** (e - bits) / 2


def assert_parity(got, want, atol=ATOL, min_cos=MIN_ROW_COS, what="", out="f32", raw=False):
    """Max-abs error <= atol and per-row cosine >= min_cos against the oracle.

    By default the error beyond the output dtype's own rounding (half an ulp of a
    16-bit output at |want|; zero for fp32) is held to atol, which matters only where
    |out| is large enough for that half-ulp to approach atol (fp16 at |out| >= 2).
    raw=True holds the raw error to atol, with no allowance: the bar as stated.
    """
    assert got.shape == want.shape, (got.shape, want.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got - want)
    excess = err - half_ulp(want, out)
    worst = np.unravel_index(np.argmax(excess), err.shape)
    cos = row_cosines(got, want)
    note(f"  parity {what}: max-abs {err.max():.3e}, max beyond {out} rounding {excess.max():.3e} "
         f"at {tuple(int(i) for i in worst)}, min row-cos {cos.min():.7f}")
    if raw:
        assert err.max() <= atol, f"{what}: max-abs error {err.max():.3e} > {atol}"
    assert excess.max() <= atol, f"{what}: error {excess.max():.3e} beyond {out} output rounding > {atol} at {worst}"
    assert cos.min() >= min_cos, f"{what}: min row cosine {cos.min():.7f} < {min_cos}"


def small(name, **kw):
    return synth.config(name, **kw)
