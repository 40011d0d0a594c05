"""Dense matrix product in float64 -- test infrastructure, not product code.

"ML-Triton, A Multi-Level Compilation and Language Extension to Triton GPU Programming",
section 2 (the tiled GEMM of the Triton tutorial that the paper compiles: a workgroup
accumulates its block of C over k-steps in a float32 accumulator and stores it once)
and section 4.1 (compute-bound GEMMs with m = 1k..16k from LLM layers):

    C[m, n] = sum_k A[m, k] * B[k, n],     A: [M, K],  B: [K, N],  C: [M, N].

Readings (listed in the design notes): A and B are row-major; the accumulation is in
float32 and C is stored in the input type (round to nearest even), as the tutorial's
kernel converts its float32 accumulator on store.  :func:`gemm` gives the exact
product (every bf16 / fp16 product is exact in float64 and the float64 sum is within
K * 2^-53 relative of the exact sum); :func:`gemm_error_bound` gives the largest error
any float32-accumulated, once-rounded result may have.
"""
from __future__ import annotations

import numpy as np

__all__ = ["gemm", "gemm_error_bound", "UNIT_ROUNDOFF"]

# Unit roundoff (half an ulp, relative) of the stored C: 2^-p for p significand bits.
UNIT_ROUNDOFF = {"bf16": 2.0 ** -8, "f16": 2.0 ** -11, "f32": 2.0 ** -24}
# Half the spacing of the subnormal numbers of each type: the absolute rounding error
# floor near zero.
_SUBNORMAL_HALF_GAP = {"bf16": 2.0 ** -134, "f16": 2.0 ** -25, "f32": 2.0 ** -150}


def gemm(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """``a [M, K] @ b [K, N]`` in float64."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    if a.ndim != 2 or b.ndim != 2 or a.shape[1] != b.shape[0]:
        raise ValueError("need a [M, K] and b [K, N]")
    return a @ b


def gemm_error_bound(a: np.ndarray, b: np.ndarray, out_dtype: str) -> np.ndarray:
    """Per-element bound on |C_computed - C| for a result accumulated in float32 (any
    order, each addition rounded) and rounded once to ``out_dtype``:

        u_out * |C| + (1 + u_out) * gamma_K * (|A| |B|) + floor,
        gamma_K = K u32 / (1 - K u32),  u32 = 2^-24,

    the standard bound for a rounded dot product (Higham, "Accuracy and Stability of
    Numerical Algorithms", section 3.1) followed by one rounding to the output type.
    """
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    K = a.shape[1]
    u32 = 2.0 ** -24
    gamma = K * u32 / (1.0 - K * u32)
    u = UNIT_ROUNDOFF[out_dtype]
    return (u * np.abs(a @ b) + (1.0 + u) * gamma * (np.abs(a) @ np.abs(b))
            + _SUBNORMAL_HALF_GAP[out_dtype])
