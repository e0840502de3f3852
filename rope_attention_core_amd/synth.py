"""Seeded synthetic inputs for the fused RoPE attention core.

This module draws the input tensors and nothing else: no rotation, no table, no
softmax. Both the HIP path and the CPU checker receive exactly the arrays made
here. The pages measure real DiT activations and SAME-L decoder activations; none
of that data exists here, so seeded normal draws with the pages' shapes stand in:

* DiT shapes: head dim 64 ("hd=64", quantize README, section "The levers"), lengths
  256, 1292 (a two-minute latent) and 4096 (about six minutes; TensorRT engines
  README, section "Benchmarks"), batch 1 per pass with CFG as a cond + uncond pair
  (sa3_trt README, section "DiT precision").
* SAME-L shape: differential attention under a sliding window (TensorRT engines
  README, sections "The SAME-L attention kernel" and "How the kernels differ"), with
  a window of 513 keys and with the kernel's own +-17 keys ("Building your own").
* Medium-DiT shape: the differential core at the long latent (the FP16-fix
  discussion, section "Compatibility": the medium DiT is the differential one). The
  pages give no head count; 24 heads as in the long-latent DiT shape.

Recipe: ``numpy.random.default_rng(seed)`` draws fp64 standard normals in the order
q, k, v (q1, k1, q2, k2, v when differential), each scaled by ``std``; the spike
rows (if any) are drawn afterwards, per (b, h), without replacement, and scaled by
``spike`` before rounding. The values are then rounded to the IO dtype: fp16 with
numpy, bf16 with torch (round to nearest even), and stored as np.float16 or as
uint16 bf16 bit patterns.
"""

from dataclasses import dataclass, replace

import numpy as np

__all__ = ["Config", "CONFIGS", "config", "make_inputs", "to_storage"]


@dataclass(frozen=True)
class Config:
    name: str
    B: int
    H: int
    L: int
    D: int
    io: str                # "f16" or "bf16"
    seed: int
    std: float = 1.0
    window: int = -1       # half-width; < 0 means full attention
    lam: float = 0.0
    diff: bool = False
    out: str = "io"        # "io", "f16", "bf16" or "f32"
    spike_frac: float = 0.0
    spike: float = 1.0
    base: float = 10000.0

    @property
    def scale(self):
        return 1.0 / float(np.sqrt(self.D))

    @property
    def out_dtype(self):
        return self.io if self.out == "io" else self.out

    def with_(self, **kw):
        return replace(self, **kw)


CONFIGS = {
    # tiny RoPE attention
    "tiny": Config("tiny", 1, 2, 64, 64, "f16", seed=1),
    # DiT short clip
    "dit_short": Config("dit_short", 1, 24, 256, 64, "f16", seed=2, std=0.5),
    # DiT two-minute latent (L = 1292 is not a tile multiple) and its prime-length twin
    "dit_2min": Config("dit_2min", 1, 24, 1292, 64, "f16", seed=3),
    "dit_2min_prime": Config("dit_2min_prime", 1, 24, 1291, 64, "f16", seed=4),
    # DiT long latent, CFG pair, bf16, 1% of K rows x8
    "dit_long": Config("dit_long", 2, 24, 4096, 64, "bf16", seed=5, out="f32",
                       spike_frac=0.01, spike=8.0),
    # SAME-L-style differential sliding-window attention, window 513 keys (w = 256)
    "samel_swa": Config("samel_swa", 1, 16, 8192, 64, "bf16", seed=6, window=256,
                        lam=0.8, diff=True, out="f32"),
    # the same with the SAME-L kernel's own window of +-17 keys (35 keys)
    "samel_w17": Config("samel_w17", 1, 16, 8192, 64, "bf16", seed=8, window=17,
                        lam=0.8, diff=True, out="f32"),
    # medium-DiT-style differential full attention at the long latent, CFG pair
    "dit_medium_diff": Config("dit_medium_diff", 2, 24, 4096, 64, "bf16", seed=7, lam=0.8,
                              diff=True, out="f32"),
    # the long latent with the same model width in 12 heads of 128
    "dit_long_d128": Config("dit_long_d128", 2, 12, 4096, 128, "bf16", seed=10, out="f32",
                            spike_frac=0.01, spike=8.0),
}


def config(name, **overrides):
    cfg = CONFIGS[name]
    return cfg.with_(**overrides) if overrides else cfg


def to_storage(x64, io):
    """Round fp64 draws to the IO dtype's storage: np.float16, or uint16 bf16 bits."""
    if io == "f16":
        return np.asarray(x64, dtype=np.float64).astype(np.float16)
    if io == "bf16":
        import torch
        t = torch.from_numpy(np.ascontiguousarray(np.asarray(x64, dtype=np.float32)))
        return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()
    raise ValueError(f"unknown io dtype {io!r}")


def make_inputs(cfg):
    """Draw the inputs of ``cfg``. Returns a dict of storage arrays.

    Plain: q, k, v each [B, H, L, D]. Differential: q and k are stacked
    [2, B, H, L, D] (branch 1 then branch 2) and v is [B, H, L, D].
    """
    rng = np.random.default_rng(cfg.seed)
    shape = (cfg.B, cfg.H, cfg.L, cfg.D)
    if cfg.diff:
        q1 = rng.standard_normal(shape) * cfg.std
        k1 = rng.standard_normal(shape) * cfg.std
        q2 = rng.standard_normal(shape) * cfg.std
        k2 = rng.standard_normal(shape) * cfg.std
        v = rng.standard_normal(shape) * cfg.std
        q = np.stack([q1, q2])
        k = np.stack([k1, k2])
        del q1, q2, k1, k2
    else:
        q = rng.standard_normal(shape) * cfg.std
        k = rng.standard_normal(shape) * cfg.std
        v = rng.standard_normal(shape) * cfg.std
    if cfg.spike_frac > 0:
        n = int(round(cfg.spike_frac * cfg.L))
        kk = k if not cfg.diff else k[0]
        for b in range(cfg.B):
            for h in range(cfg.H):
                idx = rng.choice(cfg.L, size=n, replace=False)
                kk[b, h, idx, :] *= cfg.spike
    return {"q": to_storage(q, cfg.io), "k": to_storage(k, cfg.io), "v": to_storage(v, cfg.io)}
