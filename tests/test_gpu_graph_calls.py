"""GPU: N back-to-back calls captured in one graph, every output against the oracle.

The pages' runtime captures a whole forward into one stream graph (sa3_trt README,
"Notes on the design": the full-pipeline graph), and a kernel that silently does
nothing inside such a capture goes unnoticed (TensorRT engines README, "Why JIT breaks
on sm_120"). A medium DiT forward makes 96 fused attention calls and a small one 40;
at the short latents (L = 1 ... 256) these calls are the launch-bound regime. Here
each of the 96 calls of a graph has its own seeded inputs and its own output buffer,
and cycles through plain full attention, the differential form (lambda = 0.8) and a
sliding window; the graph is replayed twice with the outputs poisoned (NaN) in
between, and every element of every output is compared with the oracle. A second
graph of the first 40 calls into fresh buffers must reproduce those outputs bitwise.
"""

import numpy as np
import pytest

from rope_attention_core_amd import synth

import gpu_common as G

pytestmark = pytest.mark.gpu

N_CALLS = 96
N_SMALL = 40


def _variant(i, L):
    """Call i's configuration: plain, differential, windowed (half-width L // 8)."""
    kind = i % 3
    seed = 20000 + 1000 * L + i
    if kind == 0:
        return synth.config("dit_short", L=L, seed=seed)
    if kind == 1:
        return synth.config("samel_swa", L=L, H=24, io="f16", out="f16", std=0.5, window=-1, seed=seed)
    return synth.config("dit_short", L=L, window=max(0, L // 8), seed=seed)


def _setup(L, n):
    torch = G.torch_mod()
    calls = []
    for i in range(n):
        cfg = _variant(i, L)
        inp = synth.make_inputs(cfg)
        q, k, v = (G.to_device(inp[nm], cfg.io) for nm in ("q", "k", "v"))
        c, s = G.device_table(cfg.L, cfg.D, cfg.base)
        out = torch.empty((cfg.B, cfg.H, cfg.L, cfg.D), dtype=torch.float16, device="cuda")
        calls.append((cfg, inp, q, k, v, c, s, out))
    return calls


def _issue(call, out=None):
    cfg, inp, q, k, v, c, s, o = call
    G.sa3.forward(q, k, v, c, s, window=cfg.window, lam=cfg.lam, scale=cfg.scale, out=o if out is None else out,
                  differential=cfg.diff)


def _capture(calls, outs):
    torch = G.torch_mod()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for call, o in zip(calls, outs):
            _issue(call, o)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for call, o in zip(calls, outs):
            _issue(call, o)
    return graph


@pytest.mark.parametrize("L", [1, 16, 64, 256])
def test_graph_of_calls_matches_oracle(L):
    torch = G.torch_mod()
    calls = _setup(L, N_CALLS)
    outs = [c[7] for c in calls]
    G.note(f"  graph: {N_CALLS} calls at L={L}, H=24")
    graph = _capture(calls, outs)
    want = [G.run_oracle(c[0], c[1]) for c in calls]
    first = None
    for rep in range(2):
        for o in outs:
            o.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = [o.float().cpu().numpy().astype(np.float64) for o in outs]
        for i, (g, w) in enumerate(zip(got, want)):
            cfg = calls[i][0]
            G.assert_parity(g, w, what=f"L={L} call {i} ({'diff' if cfg.diff else 'plain'} w={cfg.window}) "
                                      f"replay {rep}", out="f16", raw=True)
        if first is None:
            first = got
        else:
            assert all(np.array_equal(a, b) for a, b in zip(first, got)), "replays differ"

    # the small DiT's 40 calls, captured on their own into fresh buffers
    small_outs = [torch.full_like(o, float("nan")) for o in outs[:N_SMALL]]
    g40 = _capture(calls[:N_SMALL], small_outs)
    for o in small_outs:
        o.fill_(float("nan"))
    torch.cuda.synchronize()
    g40.replay()
    torch.cuda.synchronize()
    for i, o in enumerate(small_outs):
        assert np.array_equal(o.float().cpu().numpy().astype(np.float64), first[i]), f"40-call graph, call {i}"
