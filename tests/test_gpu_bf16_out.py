"""GPU: the bf16-output form of the bf16 configurations, errors in bf16 ulps.

The bf16 long-latent and SAME-L-style configurations are graded with FP32 output: a
bf16 output carries 8 significant bits, so its own rounding exceeds 2e-3 wherever
|out| >= 0.5. Here the same calls write bf16 output (the IO type, as the pages' bf16
fused MHA tier would), at full size; sampled rows are compared with the oracle and the
error is reported in units of the bf16 ulp at the oracle's value. The bar is the
arithmetic bar on top of the output's own rounding: |err| <= half an ulp + 2e-3, and
the row cosine.
"""

import numpy as np
import pytest

from rope_attention_core_amd import synth

import gpu_common as G

pytestmark = pytest.mark.gpu


def _ulp_bf16(x):
    a = np.maximum(np.abs(x), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(a)) - 7)


@pytest.mark.parametrize("name", ["dit_long", "samel_swa"])
def test_bf16_output_in_ulps(name):
    cfg = synth.config(name, out="bf16")
    inp = synth.make_inputs(cfg)
    got = G.run_gpu(cfg, inp)
    assert np.all(np.isfinite(got))
    rng = np.random.default_rng(300)
    errs, wants, gots = [], [], []
    heads = [(0, 0), (cfg.B - 1, cfg.H - 1), (0, cfg.H // 2)]
    for b, h in heads:
        rows = np.unique(np.concatenate([[0, 1, cfg.L - 1], rng.integers(0, cfg.L, 125)]))
        want = G.run_oracle_rows(cfg, inp, b, h, rows)
        g = got[b, h, rows]
        G.assert_parity(g, want, what=f"{name} bf16 out b{b} h{h}", out="bf16")
        errs.append(np.abs(g - want) / _ulp_bf16(want))
        wants.append(want)
        gots.append(g)
    e = np.concatenate([x.ravel() for x in errs])
    w = np.abs(np.concatenate([x.ravel() for x in wants]))
    big = w >= 2.0 ** -4     # where 2e-3 is below one ulp, the output's rounding dominates
    G.note(f"  {name} bf16 out: {e.size} elements; error in bf16 ulps: max {e.max():.3f}, "
           f"max where |out| >= 1/16 {e[big].max():.3f} ({big.sum()} elements), median {np.median(e):.3f}, "
           f"within 0.5 ulp {np.mean(e <= 0.5 + 1e-9):.4f}, within 1 ulp {np.mean(e <= 1.0 + 1e-9):.4f}")
    # half an ulp of rounding plus the arithmetic's ~3e-4, which is 0.6 ulp at |out| = 1/16
    assert e[big].max() <= 1.5
