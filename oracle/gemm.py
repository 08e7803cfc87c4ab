"""GEMM oracle: C = A . B in fp64.

Source: "Defeating nondeterminism in LLM inference", introduction (torch.mm of two
2048x2048 bf16 matrices) and section "batch-invariant matrix multiplication".  The
products of bf16 (or fp32) operands are exact in fp64 and the fp64 sum is far below
one bf16 ulp, so this is the plain definition.  The hardware order inside a matrix
instruction is not replayed (the arXiv abstract on cross-vendor mismatch traces
differences to exactly that order); the GPU result is graded within 1 bf16 ulp at
output scale (oracle.check) and bit-exact when the inputs make every order exact.

B is given either as [K, N] (torch.mm orientation, layout 'kn') or as a Linear
weight [N, K] (layout 'nk', C = A . B^T).
"""
from __future__ import annotations

import numpy as np

from .fp import bf16_to_f64


def gemm_f64(a, b, b_layout: str = "kn", a_dtype: str = "bf16") -> np.ndarray:
    A = bf16_to_f64(a) if a_dtype == "bf16" else np.asarray(a, dtype=np.float32).astype(np.float64)
    B = bf16_to_f64(b)
    if b_layout == "nk":
        B = B.T
    elif b_layout != "kn":
        raise ValueError(b_layout)
    return A @ B
