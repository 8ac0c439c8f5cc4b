"""Storage rounding used by the oracle (test infrastructure only).

The pages do not state a precision; the workloads store maps and outputs in
bf16 or fp32. The oracle computes in float64 and rounds once, at storage, to the
nearest representable value of the storage type, ties to even.
"""
import numpy as np


def round_bf16(x):
    """Round float64 values to the nearest bf16 value (ties to even), as float64.

    bf16 keeps 8 significant bits: for |x| in [2**(e-1), 2**e) the spacing is
    2**(e-8). Below the smallest normal bf16 (2**-126) the spacing is fixed at
    2**-133. The rounding is done directly from float64 (no float32 detour, so
    there is no double rounding).
    """
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)
    e = np.maximum(e, -125)
    q = np.ldexp(1.0, e - 8)
    with np.errstate(over="ignore", invalid="ignore"):
        r = np.rint(x / q) * q
    return np.where(np.isfinite(x), r, x)


def round_f32(x):
    """Round float64 values to the nearest float32 value (ties to even), as float64.

    numpy's float64 -> float32 conversion is the IEEE 754 one: round to nearest,
    ties to even, with float32 subnormals below 2**-126 and overflow to infinity.
    """
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)
