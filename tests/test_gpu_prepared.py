"""GPU: prepare() / PreparedCall, the binding's lean path for repeated eager calls.

A PreparedCall enqueues the call it was prepared for again with one C-ABI call; its
outputs must be bitwise those of forward() on the same tensors, on every kernel path,
after the inputs are refilled in place, and on another stream.
"""

import numpy as np
import pytest

from rope_attention_core_amd import synth

import gpu_common as G

pytestmark = pytest.mark.gpu


CASES = [
    ("dit_short", {}, {}),                                    # single-span, short sequence
    ("samel_w17", dict(H=2, L=1000), {}),                     # single-span, window 17, differential
    ("dit_2min", dict(H=3, L=1000), {}),                      # small grid: 64-row tiles + pre-pass
    ("dit_long", dict(B=1, H=24, L=3000), {}),                # long-span, pre-pass by AUTO
    ("dit_2min", dict(H=2, L=700), dict(prep="never")),       # long-span fused
    ("dit_2min", dict(H=2, L=700), dict(noalloc=True, prep="always")),
]


@pytest.mark.parametrize("name,over,kw", CASES)
def test_prepared_call_equals_forward(name, over, kw):
    torch = G.torch_mod()
    cfg = synth.config(name, seed=12000 + over.get("L", 0), **over)
    inp = synth.make_inputs(cfg)
    q, k, v = (G.to_device(inp[n], cfg.io) for n in ("q", "k", "v"))
    c, s = G.device_table(cfg.L, cfg.D, cfg.base)
    odt = G.out_torch_dtype(cfg.out_dtype)
    args = dict(window=cfg.window, lam=cfg.lam, scale=cfg.scale, differential=cfg.diff)
    fwd_kw = {k2: v2 for k2, v2 in kw.items() if k2 != "noalloc"}
    want = G.sa3.forward(q, k, v, c, s, out_dtype=odt, **args, **fwd_kw)
    call = G.sa3.prepare(q, k, v, c, s, out=torch.full_like(want, float("nan")), **args, **kw)
    got = call()
    torch.cuda.synchronize()
    assert torch.equal(got, want)
    # new inputs written in place: the prepared call sees them
    inp2 = synth.make_inputs(cfg.with_(seed=cfg.seed + 1))
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        t.copy_(G.to_device(inp2[n], cfg.io))
    want2 = G.sa3.forward(q, k, v, c, s, out_dtype=odt, **args, **fwd_kw)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        got2 = call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    assert torch.equal(got2, want2)
    assert not torch.equal(want2, want)
    rows = np.array([0, cfg.L // 2, cfg.L - 1])
    G.assert_parity(got2[0, 0, rows].float().cpu().numpy().astype(np.float64),
                    G.run_oracle_rows(cfg, inp2, 0, 0, rows), what=f"prepared {name}", out=cfg.out_dtype)
