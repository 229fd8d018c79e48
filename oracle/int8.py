"""Symmetric int8 codec and the per-token-per-head quantiser (oracle; test infrastructure).

The pages only say that FP8/INT8 quantisation keeps k_scale / v_scale buffers beside the
cache (PocketLLM "cpp_engine Batching Implementation (Phase 3.1)", "current KV cache
structure"). The reading used here mirrors the FP8 one: one fp32 scale per (token, KV
head) row equal to absmax / 127, codes = x / scale (float32 division, correctly
rounded) rounded to the nearest integer with ties to even and clamped to [-127, 127]
(-128 is never produced, so the code range is symmetric), a zero row giving scale 0 and
codes 0, and dequantisation code * scale.

Pinned by the -m "not gpu" tests: exact multiples of the scale come back exactly, ties
go to the even integer, the row's absmax maps to +-127, codes are odd under negation,
and the dequantisation error is at most half a scale step (plus float32 rounding).
"""
import numpy as np

INT8_MAX = 127.0


def round_half_even(y):
    """Nearest integer, ties to the even one (float64 result of float32 input)."""
    y = np.asarray(y, dtype=np.float64)
    fl = np.floor(y)
    frac = y - fl
    up = (frac > 0.5) | ((frac == 0.5) & (np.mod(fl, 2.0) == 1.0))
    return fl + up


def quantize_rows(x):
    """Per-row quantiser: x is float32 [..., D] (exact source values). Returns
    (codes int8 [..., D], scale float32 [...])."""
    x = np.asarray(x, dtype=np.float32)
    a = np.max(np.abs(x), axis=-1)
    scale = (a / np.float32(INT8_MAX)).astype(np.float32)
    zero = a == 0
    safe = np.where(zero, np.float32(1.0), scale).astype(np.float32)
    y = (x / safe[..., None]).astype(np.float32)
    codes = np.clip(round_half_even(y), -INT8_MAX, INT8_MAX).astype(np.int8)
    codes[zero] = 0
    scale = np.where(zero, np.float32(0.0), scale).astype(np.float32)
    return codes, scale


def dequantize(codes, scale):
    """float64 values code * scale (exact: 8 + 24 significant bits fit in 53)."""
    return np.asarray(codes, dtype=np.float64) * np.asarray(scale, dtype=np.float64)[..., None]
