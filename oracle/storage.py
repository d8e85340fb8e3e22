"""Exact decoding of stored KV/Q bit patterns to float64 (oracle; test infrastructure only).

The pages fix no precision; every storage format used here (fp32, fp16, bf16) widens to
float64 without rounding, so the oracle sees exactly the values the device holds.
"""
import numpy as np


def to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Stored array -> float64.

    f32  : numpy float32, widened exactly.
    f16  : numpy float16, widened exactly (numpy handles subnormals and specials).
    bf16 : numpy uint16 holding the upper half of an IEEE binary32; placing the 16 bits in the
           high half of a 32-bit word yields that binary32 value exactly.
    """
    a = np.asarray(a)
    if dtype == "f32":
        assert a.dtype == np.float32
        return a.astype(np.float64)
    if dtype == "f16":
        assert a.dtype == np.float16
        return a.astype(np.float64)
    if dtype == "bf16":
        assert a.dtype == np.uint16
        widened = a.astype(np.uint32) << np.uint32(16)
        return widened.view(np.float32).astype(np.float64)
    raise ValueError("unknown dtype %r" % dtype)


def scale_as_used(scale: float) -> float:
    """The kernel receives the softmax scale as a binary32; the oracle uses that same value."""
    return float(np.float32(scale))
