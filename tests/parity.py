"""The parity comparison shared by the GPU tests and the CPU power tests.

The bars are those stated for the path: slot scatter and block copy
bit-exact; decode within 1e-5 max abs for fp32, and 1e-2 for bf16 and for
e4m3/int4 caches (against the oracle on the same codes and scales).
"""
from __future__ import annotations

import numpy as np

TOL = {"f32": 1e-5, "bf16": 1e-2, "fp8": 1e-2, "int4": 1e-2}


def parity_error(got: np.ndarray, want: np.ndarray) -> float:
    """Max abs difference of two float64 output arrays (NaN or inf in `got` fails)."""
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    if got.shape != want.shape:
        raise AssertionError(f"shape {got.shape} != {want.shape}")
    if not np.isfinite(got).all():
        raise AssertionError("non-finite output")
    return float(np.abs(got - want).max()) if got.size else 0.0
