"""GPU parity of the persistent long-span kernel.

Grids of more query tiles than compute units whose query tiles span at most 32 key
tiles (sliding windows) run persistent: one workgroup per compute unit takes several
query tiles in turn and, when every tile spans >= 129 keys, its key-tile pipeline runs
on from one query tile into the next. The small shapes of the other GPU tests never
reach that path, so these cases use full-size grids (> 256 query tiles) and compare
sampled rows with the fp64 oracle: the first and last rows of query tiles (where one
item ends and the next begins), the ragged tail, and random rows, on the first and
last (b, h) slabs. Covered: the pipeline running on (window >= 128) and starting each
tile cold (window < 128), plain and differential, head dim 64 and 128 (the
differential one at 128 has no LDS to spare and always starts cold), a length that is
not a multiple of the tile, and both pre-pass policies (bitwise equal).
"""

import numpy as np
import pytest

from rope_attention_core_amd import synth

import gpu_common as G

pytestmark = pytest.mark.gpu


def _rows(L, bm, seed):
    rng = np.random.default_rng(seed)
    edges = []
    for q0 in range(0, L, bm):
        edges += [q0, q0 + 1, q0 + bm - 1]
    picks = np.concatenate([np.asarray(edges[:24] + edges[-12:], dtype=np.int64),
                            np.asarray([L - 2, L - 1], dtype=np.int64), rng.integers(0, L, 16)])
    return np.unique(np.clip(picks, 0, L - 1))


CASES = [
    # name, overrides (all > 256 query tiles, <= 32 key tiles each)
    ("samel_swa", dict(B=1, H=16, L=8192, window=256, lam=0.0, diff=False)),            # plain, runs on
    ("dit_2min", dict(B=1, H=16, L=8192, window=64)),                                   # plain f16, cold
    ("samel_swa", dict(B=1, H=16, L=4096, window=300)),                                 # differential
    ("samel_swa", dict(B=1, H=8, L=8192, window=256, D=128)),                           # diff D=128, cold
    ("dit_long", dict(B=1, H=16, L=8192, window=200, D=128)),                           # plain D=128
    ("dit_long", dict(B=1, H=16, L=8000, window=150)),                                  # ragged L
]


@pytest.mark.parametrize("name,kw", CASES)
def test_persistent_grid_sampled_parity(name, kw):
    torch = G.torch_mod()
    cfg = synth.config(name, seed=13000 + kw["L"] + kw.get("D", 64), **kw)
    inp = synth.make_inputs(cfg)
    q, k, v = (G.to_device(inp[n], cfg.io) for n in ("q", "k", "v"))
    c, s = G.device_table(cfg.L, cfg.D, cfg.base)
    G.note(f"  persistent: {name} {kw}")
    outs = {}
    for prep in ("never", "always"):
        outs[prep] = G.sa3.forward(q, k, v, c, s, window=cfg.window, lam=cfg.lam, scale=cfg.scale,
                                   out_dtype=G.out_torch_dtype(cfg.out_dtype), differential=cfg.diff, prep=prep)
    torch.cuda.synchronize()
    assert torch.equal(outs["never"], outs["always"]), "pre-pass and fused staging differ"
    bm = 128 if cfg.diff else 256
    rows = _rows(cfg.L, bm, 13100)
    for b, h in ((0, 0), (cfg.B - 1, cfg.H - 1)):
        want = G.run_oracle_rows(cfg, inp, b, h, rows)
        got = outs["never"][b, h, rows].float().cpu().numpy().astype(np.float64)
        assert np.isfinite(got).all()
        G.assert_parity(got, want, what=f"{name} {kw} (b,h)=({b},{h})", out=cfg.out_dtype)


def test_persistent_grid_in_a_graph():
    """A persistent call captured in a graph: every replay gives the eager bits."""
    torch = G.torch_mod()
    cfg = synth.config("samel_swa", B=1, H=16, L=4096, window=300, seed=13200)
    inp = synth.make_inputs(cfg)
    q, k, v = (G.to_device(inp[n], cfg.io) for n in ("q", "k", "v"))
    c, s = G.device_table(cfg.L, cfg.D, cfg.base)
    call = dict(window=cfg.window, lam=cfg.lam, scale=cfg.scale, differential=True,
                out_dtype=G.out_torch_dtype(cfg.out_dtype))
    eager = G.sa3.forward(q, k, v, c, s, **call)
    out = torch.empty_like(eager)
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        for _ in range(2):
            G.sa3.forward(q, k, v, c, s, out=out, **call)
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        G.sa3.forward(q, k, v, c, s, out=out, **call)
    for i in range(3):
        out.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {i} differs from eager"
