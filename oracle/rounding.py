"""Rounding of fp64 values to the narrow formats at the method's cast points.

Test infrastructure only (see the package header).

The method computes RoPE in FP32 and casts the result back to the activation dtype
(FP16 or BF16) before QK^T ("Fixes the medium DiT's FP16-mixed ONNX ..." discussion,
section "The bug": apply_rotary_pos_emb computes in FP32 and ends with a cast to
the output dtype). The pages do not name a rounding mode; this oracle uses IEEE
round-to-nearest-even for every cast, the IEEE default.

Parity: pinned in tests/test_oracle_rounding.py against an exact rational
(fractions.Fraction) round-to-nearest-even written independently in oracle/brute.py,
on random values, exact ties, subnormals, overflow and NaN.
"""

import numpy as np

__all__ = ["f32", "f32_to_bf16_bits", "bf16_bits_to_f64", "f32_to_f16", "widen_io", "round_io"]


def f32(x):
    """Round fp64 values to fp32 (numpy's cast is IEEE round-to-nearest-even)."""
    return np.asarray(x, dtype=np.float64).astype(np.float32)


def f32_to_bf16_bits(x32):
    """Round fp32 values to bf16, returned as uint16 bit patterns (RNE).

    bf16 is the upper half of an fp32 word; rounding to nearest-even adds
    0x7FFF plus the lowest kept bit before truncating. NaN stays NaN (quiet bit
    forced). Overflow past the largest finite bf16 goes to infinity, as IEEE
    rounding requires.
    """
    x32 = np.ascontiguousarray(np.asarray(x32, dtype=np.float32))
    u = x32.view(np.uint32).astype(np.uint64)
    keep_lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + keep_lsb) >> np.uint64(16)).astype(np.uint16)
    nan = np.isnan(x32)
    if nan.any():
        r[nan] = ((u[nan] >> np.uint64(16)) | np.uint64(0x40)).astype(np.uint16)
    return r


def bf16_bits_to_f64(bits):
    """Widen bf16 bit patterns exactly to fp64."""
    b = np.ascontiguousarray(np.asarray(bits, dtype=np.uint16))
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def f32_to_f16(x32):
    """Round fp32 values to fp16 (numpy's float32->float16 cast is RNE)."""
    return np.asarray(x32, dtype=np.float32).astype(np.float16)


def widen_io(arr, io):
    """Widen an IO-dtype storage array exactly to fp64.

    ``io`` is "f16" (storage np.float16) or "bf16" (storage uint16 bit patterns).
    """
    if io == "f16":
        return np.asarray(arr, dtype=np.float16).astype(np.float64)
    if io == "bf16":
        return bf16_bits_to_f64(arr)
    raise ValueError(f"unknown io dtype {io!r}")


def round_io(x32, io):
    """Round fp32 values to the IO dtype (RNE) and widen the result to fp64."""
    if io == "f16":
        return f32_to_f16(x32).astype(np.float64)
    if io == "bf16":
        return bf16_bits_to_f64(f32_to_bf16_bits(x32))
    raise ValueError(f"unknown io dtype {io!r}")
