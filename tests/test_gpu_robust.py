"""GPU robustness: determinism, exact pins, guard bands, graph capture, entry points.

All calls go through the C-ABI. None of these plants a fault: every buffer passed to
the library is a valid device allocation of the documented size.
"""

import ctypes

import numpy as np
import pytest

import rope_attention_core_amd as sa3
from rope_attention_core_amd import synth

import gpu_common as G

pytestmark = pytest.mark.gpu


def _dev_inputs(cfg):
    inp = synth.make_inputs(cfg)
    return inp, G.to_device(inp["q"], cfg.io), G.to_device(inp["k"], cfg.io), G.to_device(inp["v"], cfg.io)


def _fwd(cfg, q, k, v, **kw):
    c, s = G.device_table(cfg.L)
    out = sa3.forward(q, k, v, c, s, window=cfg.window, lam=cfg.lam, scale=cfg.scale,
                      out_dtype=G.out_torch_dtype(cfg.out_dtype), differential=cfg.diff, **kw)
    G.torch_mod().cuda.synchronize()
    return out


@pytest.mark.parametrize("name,kw", [("dit_2min", {}), ("dit_long", dict(H=4, L=2048)),
                                     ("samel_swa", dict(H=3, L=2500)), ("samel_w17", dict(H=3, L=3000)),
                                     ("dit_short", {})])
def test_bitwise_run_to_run_determinism(name, kw):
    cfg = synth.config(name, **kw)
    _, q, k, v = _dev_inputs(cfg)
    a = _fwd(cfg, q, k, v)
    b = _fwd(cfg, q, k, v)
    torch = G.torch_mod()
    assert torch.equal(a.view(torch.int16) if a.dtype != torch.float32 else a.view(torch.int32),
                       b.view(torch.int16) if b.dtype != torch.float32 else b.view(torch.int32))


def test_different_seeds_give_different_outputs():
    """An omitted stage would return the same bytes for every seed."""
    outs = []
    for seed in (11, 12):
        cfg = synth.config("dit_2min", H=2, L=500, seed=seed)
        _, q, k, v = _dev_inputs(cfg)
        outs.append(_fwd(cfg, q, k, v).float().cpu().numpy())
    assert np.mean(outs[0] != outs[1]) > 0.99
    assert np.all(np.isfinite(outs[0])) and np.abs(outs[0]).max() > 0


@pytest.mark.parametrize("io", ["f16", "bf16"])
def test_zero_window_returns_v_exactly(io):
    cfg = synth.config("dit_2min", H=3, L=777, window=0, io=io, out="io")
    inp, q, k, v = _dev_inputs(cfg)
    got = _fwd(cfg, q, k, v)
    assert G.torch_mod().equal(got.view(G.torch_mod().int16), v.view(G.torch_mod().int16))


@pytest.mark.parametrize("io", ["f16", "bf16"])
def test_length_one_returns_v_exactly(io):
    cfg = synth.config("dit_2min", B=2, H=5, L=1, io=io, out="io")
    _, q, k, v = _dev_inputs(cfg)
    got = _fwd(cfg, q, k, v)
    torch = G.torch_mod()
    assert torch.equal(got.view(torch.int16), v.view(torch.int16))


@pytest.mark.parametrize("name,kw", [
    ("dit_2min", dict(H=2, L=700)),                 # long-span kernel, full attention
    ("dit_2min", dict(H=2, L=1000, window=100)),    # long-span kernel, masked edge tiles
    ("dit_2min", dict(H=2, L=2100)),                # long-span kernel with the pre-pass
    ("samel_w17", dict(H=2, L=500)),                # single-span kernel, differential window
    ("dit_short", dict(H=2, L=200)),                # single-span kernel, key-split short mode
])
@pytest.mark.parametrize("io", ["f16", "bf16"])
def test_zero_queries_give_window_mean(name, kw, io):
    """Q = 0: every valid key scores exactly 0, so P = 1 and each output row is the mean
    of the V rows in its window ((1 - lambda) times it for the differential form), up to
    the FP32 accumulation of the sums."""
    import oracle
    torch = G.torch_mod()
    cfg = synth.config(name, io=io, out="f32", seed=9400 + kw["L"], **kw)
    inp, q, k, v = _dev_inputs(cfg)
    got = _fwd(cfg, torch.zeros_like(q), k, v).double().cpu().numpy()
    V = oracle.widen_io(inp["v"], io)
    L, w = cfg.L, cfg.window
    cs = np.concatenate([np.zeros(V.shape[:2] + (1, V.shape[3])), np.cumsum(V, axis=2)], axis=2)
    i = np.arange(L)
    lo = np.maximum(0, i - w) if w >= 0 else np.zeros(L, dtype=np.int64)
    hi = np.minimum(L - 1, i + w) if w >= 0 else np.full(L, L - 1)
    want = (cs[:, :, hi + 1, :] - cs[:, :, lo, :]) / (hi - lo + 1)[:, None]
    if cfg.diff:
        want = want * (1.0 - cfg.lam)
    err = np.abs(got - want).max()
    G.note(f"  q=0 {name} {kw} {io}: max-abs vs window mean {err:.2e}")
    assert err <= 1e-5 * (1.0 + np.abs(want).max())


@pytest.mark.parametrize("w", [-1, 40])
def test_differential_lambda_zero_equals_plain(w):
    """Differential at lambda = 0 is the plain core of its first branch. The two paths
    may pick different exponent bases for a tile (the differential one moves its base
    only when a P would overflow fp16), so their P round differently: they agree to
    the same bar as against the oracle, and window-edge rows (masked tiles, where both
    paths take the exact tile maximum) are covered by w = 40."""
    cfg = synth.config("samel_swa", H=2, L=900, window=w, lam=0.0)
    inp, q, k, v = _dev_inputs(cfg)
    diff = _fwd(cfg, q, k, v)
    plain_cfg = cfg.with_(diff=False)
    plain = _fwd(plain_cfg, q[0].contiguous(), k[0].contiguous(), v)
    G.torch_mod().cuda.synchronize()
    G.assert_parity(diff.float().cpu().numpy().astype(np.float64), plain.float().cpu().numpy().astype(np.float64),
                    what=f"lambda 0 vs plain, w={w}", out=cfg.out_dtype)


def test_identical_branches_give_one_minus_lambda():
    """With Q2 = Q1 and K2 = K1 both branches compute the same bits, so the output is
    x - lambda * x for x the first branch's normalised output (lambda = 0), up to the
    FP32 rounding of the subtraction."""
    cfg = synth.config("samel_swa", H=2, L=600, window=30, lam=0.8)
    inp, q, k, v = _dev_inputs(cfg)
    q2 = G.torch_mod().stack([q[0], q[0]]).contiguous()
    k2 = G.torch_mod().stack([k[0], k[0]]).contiguous()
    d = _fwd(cfg, q2, k2, v).double()
    x = _fwd(cfg.with_(lam=0.0), q2, k2, v).double()
    assert (d - 0.2 * x).abs().max().item() < 1e-6


def _embed(t, pad_elems):
    """A copy of t inside a NaN-filled buffer with pad_elems of guard on both sides."""
    torch = G.torch_mod()
    flat = torch.full((t.numel() + 2 * pad_elems,), float("nan"), dtype=t.dtype, device=t.device)
    flat[pad_elems:pad_elems + t.numel()] = t.reshape(-1)
    return flat, flat[pad_elems:pad_elems + t.numel()].view(t.shape)


@pytest.mark.parametrize("name,kw", [("dit_2min", dict(H=3, L=1291)), ("samel_swa", dict(H=2, L=1000)),
                                     ("dit_long", dict(H=2, L=333)),
                                     # the narrow-window kernel stages keys from q0 - w, before
                                     # the slab for the first block: the guard must not leak in
                                     ("samel_w17", dict(H=2, L=1000)), ("dit_2min", dict(H=2, L=500, window=5)),
                                     ("dit_short", dict(L=200)), ("samel_swa", dict(H=2, L=100))])
def test_nan_guard_bands(name, kw):
    """Inputs and output embedded in NaN-poisoned buffers: results unchanged, guards intact."""
    torch = G.torch_mod()
    cfg = synth.config(name, **kw)
    _, q, k, v = _dev_inputs(cfg)
    clean = _fwd(cfg, q, k, v)
    pad = 4096
    _, qg = _embed(q, pad)
    _, kg = _embed(k, pad)
    _, vg = _embed(v, pad)
    c, s = G.device_table(cfg.L)
    # a table longer than L whose extra rows are NaN: only rows < L may be read
    cg = torch.full((cfg.L + 64, 32), float("nan"), device="cuda")
    sg = torch.full((cfg.L + 64, 32), float("nan"), device="cuda")
    cg[:cfg.L] = c
    sg[:cfg.L] = s
    dt = G.out_torch_dtype(cfg.out_dtype)
    oflat = torch.full((clean.numel() + 2 * pad,), float("nan"), dtype=dt, device="cuda")
    og = oflat[pad:pad + clean.numel()].view(clean.shape)
    sa3.forward(qg, kg, vg, cg, sg, window=cfg.window, lam=cfg.lam, scale=cfg.scale, out=og,
                differential=cfg.diff)
    torch.cuda.synchronize()
    assert torch.equal(og, clean)
    assert torch.isnan(oflat[:pad]).all() and torch.isnan(oflat[pad + clean.numel():]).all()


@pytest.mark.parametrize("name,kw", [("dit_short", {}), ("samel_swa", dict(H=2, L=700)),
                                     ("samel_w17", dict(H=2, L=900))])
def test_graph_capture_replays_match_eager(name, kw):
    torch = G.torch_mod()
    cfg = synth.config(name, **kw)
    _, q, k, v = _dev_inputs(cfg)
    c, s = G.device_table(cfg.L)
    eager = _fwd(cfg, q, k, v)
    out = torch.empty_like(eager)
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        for _ in range(2):  # warm up on the capture stream
            sa3.forward(q, k, v, c, s, window=cfg.window, lam=cfg.lam, scale=cfg.scale, out=out,
                        differential=cfg.diff)
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        sa3.forward(q, k, v, c, s, window=cfg.window, lam=cfg.lam, scale=cfg.scale, out=out,
                    differential=cfg.diff)
    for i in range(4):
        out.zero_()
        _ = (q.float().sum() if i % 2 else None)  # unrelated eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {i} differs from eager"


@pytest.mark.parametrize("io", ["f16", "bf16"])
@pytest.mark.parametrize("lam", [0.0, 0.8])
def test_short_entry_points_match_ex(io, lam):
    torch = G.torch_mod()
    diff = lam != 0.0
    cfg = synth.config("samel_swa", H=2, L=400, window=50, lam=lam, diff=diff, io=io, out="io")
    _, q, k, v = _dev_inputs(cfg)
    ex = _fwd(cfg, q, k, v)
    c, s = G.device_table(cfg.L)
    out = torch.empty_like(ex)
    sa3.forward_short(q, k, v, c, s, out, window=cfg.window, lam=lam, scale=cfg.scale)
    torch.cuda.synchronize()
    assert torch.equal(out, ex)


def test_errors_leave_out_untouched_on_gpu():
    torch = G.torch_mod()
    lib = sa3.load_library()
    cfg = synth.config("dit_2min", H=2, L=100)
    _, q, k, v = _dev_inputs(cfg)
    c, s = G.device_table(cfg.L)
    out = torch.full_like(v, 7.0)
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    f = lib.sa3attn_forward
    assert f(P(q), P(k), P(v), P(c), P(s), P(out), 1, 2, 100, 96, -1, 0.0, 0.125, stream) == -3
    assert f(P(q), P(k), P(v), P(c), P(s), P(out), 1, 2, 100, 64, -1, 0.0, float("nan"), stream) == -4
    assert f(P(q), P(k), P(v), P(c), P(s), P(q), 1, 2, 100, 64, -1, 0.0, 0.125, stream) == -4
    assert f(None, P(k), P(v), P(c), P(s), P(out), 1, 2, 100, 64, -1, 0.0, 0.125, stream) == -1
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())
    with pytest.raises(sa3.SA3Error):
        sa3.forward(q, k, v, c, s, scale=float("inf"), out=out)
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())
