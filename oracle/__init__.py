"""fp64 CPU oracle for the fused RoPE attention core of the Stable Audio 3 transformers.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or execute
anything in this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it. It shares no code, table, constant or
helper with the HIP library under ``rope_attention_core_amd/``; it receives the same
input arrays as plain data and computes its own RoPE table.

What it computes (the method, restated from the pages):

* RoPE is applied to Q and K in FP32 and the result is cast back to the activation
  dtype before QK^T ("Fixes the medium DiT's FP16-mixed ONNX ..." discussion,
  sections "The bug" and "The fix"; sa3_trt README, section "DiT precision").
* The cos/sin table is computed on the host in FP32 (sa3_trt README, section
  "DiT precision", the fp8 tier's baked table).
* Attention is softmax(scale * Q K^T + M) V with the softmax accumulated in FP32
  (same discussion, section "The bug"), where M masks |i - j| > w for a sliding
  window of half-width w (TensorRT engines README, section "Building your own").
* The differential variant subtracts lambda times a second softmax attention that
  shares V (TensorRT engines README, section "How the kernels differ").

Two modes share one code path:

* ``def`` mode: pure mathematics in fp64 (RoPE in fp64, no rounding anywhere).
* ``method`` mode: identical, except at the two rounding points the method itself
  defines: the rotation is evaluated in FP32 with the FP32 table and rounded
  (round-to-nearest-even) to the IO dtype. Everything after the cast-back is fp64.

Modules:
  rounding  -- fp32 / fp16 / bf16 rounding of arrays (numpy)
  rope      -- frequencies, FP32 table, rotations in both modes
  attention -- masked softmax attention, plain and differential, both modes
  brute     -- pure-Python brute force (math.fsum, exact Fractions) for tiny inputs

Parity status per function is stated in each module header.
"""

from .rounding import (
    f32,
    f32_to_bf16_bits,
    bf16_bits_to_f64,
    f32_to_f16,
    widen_io,
    round_io,
)
from .rope import (
    rope_frequencies,
    rope_angles,
    rope_table_f32,
    rope_table_bf16_angle,
    rotate_def,
    rotate_f32,
    rotate_method,
)
from .attention import (
    masked_attention,
    attn_def,
    attn_method,
    attn_method_rows,
    softmax_rows,
)

__all__ = [
    "f32", "f32_to_bf16_bits", "bf16_bits_to_f64", "f32_to_f16", "widen_io", "round_io",
    "rope_frequencies", "rope_angles", "rope_table_f32", "rope_table_bf16_angle",
    "rotate_def", "rotate_f32", "rotate_method",
    "masked_attention", "attn_def", "attn_method", "attn_method_rows", "softmax_rows",
]
