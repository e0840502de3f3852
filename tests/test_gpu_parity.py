"""GPU parity: the HIP path (through the C-ABI) against the fp64 method-mode oracle.

Bar: max-abs error <= 2e-3 and per-row cosine >= 0.99995 on the same seeded inputs,
for FP16/BF16 inputs. Small configurations are compared element by element on every
output; the full-size DiT-long and SAME-L-style configurations run on the GPU at full
size, in the launch configuration the benchmark times, and are compared on sampled
rows that the oracle computes one by one.
"""

import numpy as np
import pytest

from rope_attention_core_amd import synth

import gpu_common as G

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["tiny", "dit_short", "dit_2min", "dit_2min_prime"])
def test_config_full_parity(name):
    """The fp16-output configurations, every element: the raw max-abs error (fp16
    output rounding included) <= 2e-3 and row cosine >= 0.99995."""
    cfg = synth.config(name)
    inp = synth.make_inputs(cfg)
    got = G.run_gpu(cfg, inp)
    want = G.run_oracle(cfg, inp)
    G.assert_parity(got, want, what=name, out=cfg.out_dtype, raw=True)


def test_dit_long_full_size_sampled():
    """B=2, H=24, L=4096 bf16, 1% of K rows x8, fp32 out: every row of 3 heads sampled."""
    cfg = synth.config("dit_long")
    inp = synth.make_inputs(cfg)
    got = G.run_gpu(cfg, inp)
    assert np.all(np.isfinite(got))
    rng = np.random.default_rng(100)
    for b, h in ((0, 0), (1, 23), (0, 13)):
        rows = np.unique(np.concatenate([np.arange(0, 8), np.arange(4088, 4096), rng.integers(0, 4096, 240)]))
        want = G.run_oracle_rows(cfg, inp, b, h, rows)
        G.assert_parity(got[b, h, rows], want, what=f"dit_long b{b} h{h}")


def test_dit_long_one_head_full():
    cfg = synth.config("dit_long", B=1, H=2)
    inp = synth.make_inputs(cfg)
    G.assert_parity(G.run_gpu(cfg, inp), G.run_oracle(cfg, inp), what="dit_long H2")


def test_samel_swa_full_size_sampled():
    """B=1, H=16, L=8192 bf16 differential, w=256 (513 keys), lambda=0.8, fp32 out."""
    cfg = synth.config("samel_swa")
    inp = synth.make_inputs(cfg)
    got = G.run_gpu(cfg, inp)
    assert np.all(np.isfinite(got))
    rng = np.random.default_rng(101)
    for h in (0, 7, 15):
        rows = np.unique(np.concatenate([np.arange(0, 300), np.arange(7890, 8192), rng.integers(0, 8192, 400)]))
        want = G.run_oracle_rows(cfg, inp, 0, h, rows)
        G.assert_parity(got[0, h, rows], want, what=f"samel_swa h{h}")


def test_samel_swa_reduced_full():
    cfg = synth.config("samel_swa", H=2, L=3000)
    inp = synth.make_inputs(cfg)
    G.assert_parity(G.run_gpu(cfg, inp), G.run_oracle(cfg, inp), what="samel_swa H2 L3000")


def test_samel_w17_full_size_sampled():
    """B=1, H=16, L=8192 bf16 differential, w=17 (35 keys), lambda=0.8, fp32 out."""
    cfg = synth.config("samel_w17")
    inp = synth.make_inputs(cfg)
    got = G.run_gpu(cfg, inp)
    assert np.all(np.isfinite(got))
    rng = np.random.default_rng(102)
    for h in (0, 9, 15):
        rows = np.unique(np.concatenate([np.arange(0, 100), np.arange(8092, 8192), rng.integers(0, 8192, 400)]))
        want = G.run_oracle_rows(cfg, inp, 0, h, rows)
        G.assert_parity(got[0, h, rows], want, what=f"samel_w17 h{h}")


def test_samel_w17_reduced_full():
    cfg = synth.config("samel_w17", H=2, L=2500)
    inp = synth.make_inputs(cfg)
    G.assert_parity(G.run_gpu(cfg, inp), G.run_oracle(cfg, inp), what="samel_w17 H2 L2500")


def test_dit_medium_diff_full_size_sampled():
    """B=2, H=24, L=4096 bf16 differential full attention, lambda=0.8, fp32 out."""
    cfg = synth.config("dit_medium_diff")
    inp = synth.make_inputs(cfg)
    got = G.run_gpu(cfg, inp)
    assert np.all(np.isfinite(got))
    rng = np.random.default_rng(103)
    for b, h in ((0, 0), (1, 23), (1, 5)):
        rows = np.unique(np.concatenate([np.arange(0, 8), np.arange(4088, 4096), rng.integers(0, 4096, 120)]))
        want = G.run_oracle_rows(cfg, inp, b, h, rows)
        G.assert_parity(got[b, h, rows], want, what=f"dit_medium_diff b{b} h{h}")


def test_dit_medium_diff_one_head_full():
    cfg = synth.config("dit_medium_diff", B=1, H=1, L=2048)
    inp = synth.make_inputs(cfg)
    G.assert_parity(G.run_gpu(cfg, inp), G.run_oracle(cfg, inp), what="dit_medium_diff H1 L2048")


TAILS = [1, 2, 3, 15, 16, 17, 31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 256, 257, 511, 513, 1291, 1292,
         2047, 4093, 4095]


@pytest.mark.parametrize("L", TAILS)
def test_tail_lengths_f16(L):
    cfg = synth.config("dit_2min", H=3, L=L, seed=1000 + L)
    inp = synth.make_inputs(cfg)
    G.assert_parity(G.run_gpu(cfg, inp), G.run_oracle(cfg, inp), what=f"tail L{L}", out=cfg.out_dtype)


@pytest.mark.parametrize("L", [1, 17, 64, 65, 200, 257, 1291])
def test_tail_lengths_bf16_windowed_diff(L):
    cfg = synth.config("samel_swa", H=2, L=L, window=17, seed=2000 + L)
    inp = synth.make_inputs(cfg)
    G.assert_parity(G.run_gpu(cfg, inp), G.run_oracle(cfg, inp), what=f"swa tail L{L}")


@pytest.mark.parametrize("L", [1, 31, 64, 65, 100, 128, 129, 200, 256])
@pytest.mark.parametrize("w", [-1, 40])
def test_short_sequences_differential(L, w):
    """Short sequences (the single-span kernel) in the two-branch form, full and windowed."""
    cfg = synth.config("samel_swa", H=3, L=L, window=w, seed=7000 + L)
    inp = synth.make_inputs(cfg)
    G.assert_parity(G.run_gpu(cfg, inp), G.run_oracle(cfg, inp), what=f"short diff L{L} w{w}")


@pytest.mark.parametrize("L", [40, 129, 200, 256])
@pytest.mark.parametrize("w", [0, 5, 33, 100])
def test_short_sequences_windowed(L, w):
    cfg = synth.config("dit_short", H=2, L=L, window=w, seed=7500 + L + w)
    inp = synth.make_inputs(cfg)
    G.assert_parity(G.run_gpu(cfg, inp), G.run_oracle(cfg, inp), what=f"short w{w} L{L}", out=cfg.out_dtype)


@pytest.mark.parametrize("w", [0, 1, 15, 16, 17, 31, 32, 33, 63, 64, 65, 255, 256, 257, 698, 699, 700, 5000, -1])
@pytest.mark.parametrize("io", ["f16", "bf16"])
def test_window_sweep(w, io):
    cfg = synth.config("dit_2min", H=2, L=700, window=w, io=io, seed=3000 + max(w, 0),
                       out="f32" if io == "bf16" else "io")
    inp = synth.make_inputs(cfg)
    G.assert_parity(G.run_gpu(cfg, inp), G.run_oracle(cfg, inp), what=f"window {w} {io}", out=cfg.out_dtype)


@pytest.mark.parametrize("w", [0, 1, 16, 17, 31, 32])
def test_differential_narrow_window_sweep(w):
    """Differential windows of the single-span kernel: each wave computes the three
    32-key blocks of the span from its own row offset, whose last needed key (offset
    32 wq + 31 + 2w) lies in the third block from w = 17 and at its last key at w = 32."""
    cfg = synth.config("samel_swa", H=2, L=700, window=w, seed=4100 + w, out="f32")
    inp = synth.make_inputs(cfg)
    G.assert_parity(G.run_gpu(cfg, inp), G.run_oracle(cfg, inp), what=f"diff narrow w{w}")


@pytest.mark.parametrize("lam", [0.0, 0.8, -0.5])
@pytest.mark.parametrize("w", [-1, 17, 256])
@pytest.mark.parametrize("io", ["f16", "bf16"])
def test_differential(lam, w, io):
    cfg = synth.config("samel_swa", H=2, L=1000, window=w, lam=lam, io=io, seed=4000,
                       out="f32")
    inp = synth.make_inputs(cfg)
    G.assert_parity(G.run_gpu(cfg, inp), G.run_oracle(cfg, inp), what=f"diff lam{lam} w{w} {io}")


@pytest.mark.parametrize("io,out", [("f16", "f16"), ("f16", "bf16"), ("f16", "f32"),
                                    ("bf16", "f16"), ("bf16", "bf16"), ("bf16", "f32")])
def test_out_dtypes(io, out):
    cfg = synth.config("dit_2min", H=2, L=333, io=io, out=out, std=0.5, seed=5000)
    inp = synth.make_inputs(cfg)
    got, want = G.run_gpu(cfg, inp), G.run_oracle(cfg, inp)
    # a bf16 output carries 8 significant bits: its rounding alone moves the row cosine
    G.assert_parity(got, want, what=f"{io}->{out}", out=out, min_cos=0.9999 if out == "bf16" else G.MIN_ROW_COS)


@pytest.mark.parametrize("scale", [-0.125, 0.0, 0.37])
def test_scale_values(scale):
    cfg = synth.config("dit_2min", H=2, L=300, seed=6000)
    inp = synth.make_inputs(cfg)
    q, k, v = G.widen(inp, cfg)
    import oracle
    c32, s32 = oracle.rope_table_f32(cfg.L, 64)
    want = oracle.attn_method(q, k, v, c32, s32, "f16", scale)
    torch = G.torch_mod()
    c, s = G.device_table(cfg.L)
    import rope_attention_core_amd as sa3
    out = sa3.forward(G.to_device(inp["q"], "f16"), G.to_device(inp["k"], "f16"), G.to_device(inp["v"], "f16"),
                      c, s, scale=scale)
    torch.cuda.synchronize()
    G.assert_parity(out.float().cpu().numpy().astype(np.float64), want, what=f"scale {scale}", out="f16")


def _sampled_rows(L, seed, extra=()):
    rng = np.random.default_rng(seed)
    edges = [0, 1, 2, 17, 63, 64, 255, 256, L // 2, L - 257, L - 65, L - 18, L - 2, L - 1]
    picks = np.concatenate([np.asarray(edges, dtype=np.int64), np.asarray(list(extra), dtype=np.int64),
                            rng.integers(0, L, 24)])
    return np.unique(np.clip(picks, 0, L - 1))


@pytest.mark.parametrize("w", [17, 256])
def test_long_sequence_windowed_sampled(w):
    """L = 131072 (16x the SAME-L shape; 32-bit row offsets well above 2^24 bytes) in
    the differential windowed form: the single-span kernel (w = 17) and the long-span
    kernel with its pre-pass (w = 256), sampled rows against the oracle."""
    L = 1 << 17
    cfg = synth.config("samel_swa", H=1, L=L, window=w, seed=8100 + w)
    inp = synth.make_inputs(cfg)
    got = G.run_gpu(cfg, inp)
    rows = _sampled_rows(L, 8150 + w)
    want = G.run_oracle_rows(cfg, inp, 0, 0, rows)
    G.assert_parity(got[0, 0, rows], want, what=f"L=2^17 w={w}", out=cfg.out_dtype)


def test_long_sequence_full_sampled():
    """Full attention at L = 16384 (4x the long latent; 64 query tiles per head, the
    pre-pass on), bf16 with spiked keys, sampled rows against the oracle."""
    L = 1 << 14
    cfg = synth.config("dit_long", B=1, H=2, L=L, seed=8200)
    inp = synth.make_inputs(cfg)
    got = G.run_gpu(cfg, inp)
    for h in range(cfg.H):
        rows = _sampled_rows(L, 8250 + h)
        want = G.run_oracle_rows(cfg, inp, 0, h, rows)
        G.assert_parity(got[0, h, rows], want, what=f"L=2^14 full h{h}", out=cfg.out_dtype)
