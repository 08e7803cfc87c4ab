"""RMSNorm oracle.

Source: "Defeating nondeterminism in LLM inference", section "batch-invariant
RMSNorm": y = x * rsqrt(mean(x**2)) * weight, reduced over the hidden dimension
with an order that never depends on the batch size.

Readings (the page prints no eps and no rounding points):
  * eps goes inside the square root: r = 1 / sqrt(mean(x^2) + eps);
  * rsqrt is two correctly rounded fp32 operations, sqrt then divide;
  * the multiplies follow the page's left-to-right order: (x * r) * weight,
    then one round-to-nearest-even to bf16;
  * the sum of squares uses the fixed tree of ``oracle.tree`` with 8-element
    vectors (16-byte bf16 loads) or 4-element vectors for fp32 input.
"""
from __future__ import annotations

import numpy as np

from .fp import bf16_to_f32, f32_to_bf16, bf16_to_f64
from .tree import tree_sum


def _prep(x, in_dtype):
    if in_dtype == "bf16":
        return bf16_to_f32(x), 8
    return np.asarray(x, dtype=np.float32), 4


def rmsnorm_tree(x, gamma_bits, eps: float, in_dtype: str = "bf16", out_dtype: str = "bf16"):
    """Bit-exact replay.  x: [M, D] bf16 bits (or float32 when in_dtype='f32');
    gamma: [D] bf16 bits.  Returns bf16 bits [M, D] (or float32 when out_dtype='f32')."""
    xf, width = _prep(x, in_dtype)
    m, d = xf.shape
    g = bf16_to_f32(gamma_bits)
    sq = xf * xf                                   # exact for bf16 input; rounded for fp32
    ssum = tree_sum(sq, width)
    mean = ssum / np.float32(d)
    v = mean + np.float32(eps)
    r = np.float32(1.0) / np.sqrt(v)
    y = (xf * r[:, None]) * g[None, :]
    return f32_to_bf16(y) if out_dtype == "bf16" else y.astype(np.float32)


def rmsnorm_f64(x_bits, gamma_bits, eps: float) -> np.ndarray:
    """Plain fp64 definition (for the 1-ulp sanity pin)."""
    x = bf16_to_f64(x_bits)
    g = bf16_to_f64(gamma_bits)
    r = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    return x * r * g
