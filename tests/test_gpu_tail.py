"""GPU checks of the split tail of the long-span kernel (with the pre-pass workspace).

A grid of one 8-wave workgroup per query tile whose last round would hold at most half
as many tiles as compute units splits each of those tiles into k key ranges; the last
range to finish merges the ranges' partial (O, m, l) from the workspace. Cases: the
long latent at head dim 128 (384 tiles on 256 CUs: 256 whole, 128 split in two), grids
of fewer tiles than half the CUs (every tile split in up to four), a plain D = 64 grid
with a 32-tile tail, a wide window, a differential call, large bf16 V values in split
tiles (the guard's shift differs between ranges), run-to-run bits, the "only" /
"reuse" pair (the counters clear themselves), and graph replays. Every result is
compared with the oracle; the split changes the order of the sums over a row's keys,
so bits are compared only between calls of the same path.
"""

import numpy as np
import pytest

from rope_attention_core_amd import synth

import gpu_common as G

pytestmark = pytest.mark.gpu


def _kv_bytes(cfg):
    return (3 if cfg.diff else 2) * cfg.B * cfg.H * ((cfg.L + 63) // 64 * 64) * cfg.D * 2


def _ws_bytes(cfg, prep="always"):
    return G.sa3.workspace_bytes(cfg.B, cfg.H, cfg.L, cfg.D, window=cfg.window, differential=cfg.diff, prep=prep)


def _tiles(cfg):
    bm = 128 if cfg.diff else 256
    return (cfg.L + bm - 1) // bm, bm


def _dev(cfg, inp):
    return tuple(G.to_device(inp[n], cfg.io) for n in ("q", "k", "v"))


def _call(cfg, q, k, v, **kw):
    c, s = G.device_table(cfg.L, cfg.D, cfg.base)
    return G.sa3.forward(q, k, v, c, s, window=cfg.window, lam=cfg.lam, scale=cfg.scale,
                         out_dtype=G.out_torch_dtype(cfg.out_dtype), differential=cfg.diff, **kw)


def _split_heads(cfg, n_cu=256):
    """(b, h) pairs whose tiles include split ones (the last tiles in b*h order)."""
    nq, _ = _tiles(cfg)
    items = nq * cfg.B * cfg.H
    first = items - items % n_cu
    return sorted({divmod(lid // nq, cfg.H) for lid in range(first, items)})


def _rows(cfg, rng, n=12):
    _, bm = _tiles(cfg)
    edges = [0, 1, cfg.L - 1] + [t * bm + d for t in range(1, (cfg.L + bm - 1) // bm) for d in (-1, 0)]
    return np.unique(np.clip(np.concatenate([edges, rng.integers(0, cfg.L, n)]), 0, cfg.L - 1))


def cfg_seed(kw):
    return kw.get("L", 0) + kw.get("H", 0)


SHAPES = [
    # name, overrides: all with a split tail on 256 compute units
    ("dit_long_d128", {}),                                         # 384 tiles: 256 + 128 x 2
    ("dit_long", dict(B=1, H=24, L=3000)),                         # 288 tiles: 256 + 32 x 4
    ("dit_long", dict(B=1, H=20, L=4096, window=1500)),            # 320 tiles of 52 key tiles: 256 + 64 x 4
    ("dit_long_d128", dict(B=1, H=4, L=1500)),                     # 24 tiles, all split in 4
    ("samel_swa", dict(H=2, L=1000, window=-1)),                   # differential: 16 tiles, all split in 4
    ("samel_swa", dict(H=3, L=2000, window=400)),                  # differential window: 48 tiles x 2
]


@pytest.mark.parametrize("name,kw", SHAPES)
def test_split_tail_parity(name, kw):
    torch = G.torch_mod()
    cfg = synth.config(name, seed=15000 + cfg_seed(kw), **kw)
    assert _ws_bytes(cfg) > _kv_bytes(cfg), "the split tail does not apply to this shape"
    inp = synth.make_inputs(cfg)
    q, k, v = _dev(cfg, inp)
    G.note(f"  tail: {name} {kw}")
    got = _call(cfg, q, k, v, prep="always")
    again = _call(cfg, q, k, v, prep="always")
    torch.cuda.synchronize()
    assert torch.equal(got, again), "two calls of the split path differ"
    g = got.float().cpu().numpy().astype(np.float64)
    assert np.isfinite(g).all()
    if cfg.B * cfg.H * cfg.L <= 8 * 1000:
        G.assert_parity(g, G.run_oracle(cfg, inp), what=f"{name} {kw} split tail", out=cfg.out_dtype)
        return
    rng = np.random.default_rng(15100)
    heads = _split_heads(cfg)
    picks = [(0, 0), heads[0], heads[len(heads) // 2], heads[-1]]
    for b, h in picks:
        rows = _rows(cfg, rng)
        want = G.run_oracle_rows(cfg, inp, b, h, rows)
        G.assert_parity(g[b, h, rows], want, what=f"{name} {kw} (b,h)=({b},{h})", out=cfg.out_dtype)


def test_split_tail_full_heads():
    """The long latent at D = 128: every element of every head whose tiles were split,
    through the split path (AUTO) and the fused path (no pre-pass), against the oracle.
    (The two paths put the lazy softmax bases of a row in different places, so P rounds
    to fp16 differently: they differ by up to ~7e-4 at the spiked keys, each within the
    bar of the exact result.)"""
    torch = G.torch_mod()
    cfg = synth.config("dit_long_d128")
    inp = synth.make_inputs(cfg)
    q, k, v = _dev(cfg, inp)
    a = _call(cfg, q, k, v, prep="auto")
    f = _call(cfg, q, k, v, prep="never")
    torch.cuda.synchronize()
    rows = np.arange(cfg.L)
    for b, h in _split_heads(cfg):
        want = G.run_oracle_rows(cfg, inp, b, h, rows)
        for what, got in (("split", a), ("fused", f)):
            G.assert_parity(got[b, h].float().cpu().numpy().astype(np.float64), want,
                            what=f"dit_long_d128 (b,h)=({b},{h}) {what}", out=cfg.out_dtype)


def test_split_tail_large_v_in_split_tiles():
    """bf16 V with values near 3e38 in heads whose tiles are split: the guard redoes the
    affected ranges with their own shifts, and the merge brings them to a common one."""
    cfg = synth.config("dit_long", B=1, H=24, L=3000, seed=15200, spike_frac=0.0, out="f32")
    inp = synth.make_inputs(cfg)
    v = (inp["v"].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    heads = _split_heads(cfg)
    b, h = heads[len(heads) // 2]
    v[b, h, 2900, 3] = 3.0e38          # in the last key range of this head's split tiles
    v[b, h, 100, 7] = -1.0e6           # in the first
    v[b, h, 1500:1530, :] *= 2.0 ** 17
    big = dict(inp, v=synth.to_storage(v, "bf16"))
    q, k, vv = _dev(cfg, big)
    got = _call(cfg, q, k, vv, prep="always").float().cpu().numpy().astype(np.float64)
    assert np.isfinite(got).all()
    vmax = np.abs(v[b, h]).max()
    rows = _rows(cfg, np.random.default_rng(15201))
    want = G.run_oracle_rows(cfg, big, b, h, rows)
    G.assert_parity(got[b, h, rows], want, atol=2e-3 * vmax, min_cos=G.MIN_ROW_COS, what="split tail, large V")
    # a head without large values is unaffected
    b2, h2 = heads[0]
    rows2 = _rows(cfg, np.random.default_rng(15202), n=4)
    G.assert_parity(got[b2, h2, rows2], G.run_oracle_rows(cfg, big, b2, h2, rows2), what="split tail, other head")


def test_split_tail_only_then_reuse_and_graph():
    """The counters are cleared by the pre-pass and by the range that merges: "reuse"
    calls after one "only" call, and replays of a captured pre-pass + attention pair,
    all give the bits of an eager "always" call."""
    torch = G.torch_mod()
    cfg = synth.config("dit_long_d128", B=1, H=4, L=1500, seed=15300)
    inp = synth.make_inputs(cfg)
    q, k, v = _dev(cfg, inp)
    eager = _call(cfg, q, k, v, prep="always")
    nb = _ws_bytes(cfg)
    ws = torch.full((nb,), 0xFF, dtype=torch.uint8, device="cuda")
    out = torch.empty_like(eager)
    _call(cfg, q, k, v, prep="only", workspace=ws, out=out)
    for i in range(3):
        out.fill_(float("nan"))
        _call(cfg, q, k, v, prep="reuse", workspace=ws, out=out)
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"reuse call {i}"
    c, s = G.device_table(cfg.L, cfg.D, cfg.base)
    call = dict(window=cfg.window, lam=cfg.lam, scale=cfg.scale, out=out, differential=cfg.diff, prep="always",
                workspace=ws)
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        for _ in range(2):
            G.sa3.forward(q, k, v, c, s, **call)
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        G.sa3.forward(q, k, v, c, s, **call)
    for i in range(3):
        out.zero_()
        ws.fill_(0xFF if i % 2 else 0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {i}"
    G.assert_parity(out.float().cpu().numpy().astype(np.float64), G.run_oracle(cfg, inp), what="reused split tail",
                    out=cfg.out_dtype)
