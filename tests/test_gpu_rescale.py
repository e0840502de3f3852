"""GPU parity where the online softmax has to move its exponent base many times.

The kernels keep one exponent base per row and move it only when a tile's maximum
rises more than a fixed margin above it, rescaling O and the running sum by the
factor between the bases (single-span kernels take one exact maximum over the whole
span instead). With the unit-variance inputs of the other tests the base settles on
the first tile and almost never moves again, so these cases shape the keys so that it
must: key norms rising along the sequence (the maximum climbs tile after tile),
falling (the first tile holds the largest scores and every later P is small), and
one huge late key (a single jump of tens of powers of two at the last tiles). Each
case is compared with the fp64 oracle element by element, on the long-span kernel
with and without the pre-pass, on the single-span kernel, plain and differential,
windowed, head dim 64 and 128.
"""

import numpy as np
import pytest

from rope_attention_core_amd import synth

import gpu_common as G

pytestmark = pytest.mark.gpu


def _shaped_inputs(cfg, profile):
    inp = synth.make_inputs(cfg)
    q, k, v = G.widen(inp, cfg)
    L = cfg.L
    pos = np.arange(L, dtype=np.float64) / max(L - 1, 1)
    if profile == "rising":
        gain = 1.0 + 7.0 * pos
    elif profile == "falling":
        gain = 8.0 - 7.0 * pos
    elif profile == "late_spike":
        gain = np.ones(L)
        gain[max(L - 3, 0)] = 40.0
    else:
        raise ValueError(profile)
    k = k * gain[:, None]
    q = q * 1.5
    inp["q"] = synth.to_storage(q, cfg.io)
    inp["k"] = synth.to_storage(k, cfg.io)
    return inp


CASES = [
    # name, overrides, prep policy (long-span kernel) or None (single-span kernel)
    ("dit_2min", dict(H=2, L=1000), "never"),
    ("dit_2min", dict(H=2, L=1000), "always"),
    ("dit_2min", dict(H=2, L=1000, io="bf16", window=200), "never"),
    ("samel_swa", dict(H=2, L=900, window=-1), "never"),
    ("samel_swa", dict(H=2, L=900, window=-1), "always"),
    ("dit_2min", dict(H=2, L=700, D=128), "never"),
    ("dit_2min", dict(H=2, L=700, D=128), "always"),
    ("dit_2min", dict(H=2, L=256), None),
    ("samel_swa", dict(H=2, L=600, window=17), None),
]


@pytest.mark.parametrize("profile", ["rising", "falling", "late_spike"])
@pytest.mark.parametrize("name,kw,prep", CASES)
def test_base_moves_match_oracle(name, kw, prep, profile):
    cfg = synth.config(name, seed=12000 + kw.get("L", 0) + kw.get("D", 0), **kw)
    inp = _shaped_inputs(cfg, profile)
    G.note(f"  rescale: {name} {kw} prep={prep} {profile}")
    extra = {} if prep is None else dict(prep=prep)
    got = G.run_gpu(cfg, inp, **extra)
    want = G.run_oracle(cfg, inp)
    assert np.isfinite(got).all()
    G.assert_parity(got, want, what=f"{profile} {name} {kw} prep={prep}", out=cfg.out_dtype)
