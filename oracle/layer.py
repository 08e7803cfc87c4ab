"""Decoder-layer pieces of the oracle (Mistral-7B-shaped composition).

The pointwise steps around the three reductions ("Defeating nondeterminism in LLM
inference", section on making kernels batch-invariant: pointwise operations are
batch-invariant as long as every element runs the same code):

  RoPE    : rotate-half pairing (i, i + D/2), angle p * base^(-2i/D), i < D/2
  SwiGLU  : silu(g) * u = g / (1 + exp(-g)) * u
  residual: h + f(h)

Readings (the pages name these steps but print no formula): rotate-half pairing,
base 10000, angles in fp64.
"""
from __future__ import annotations

import numpy as np


def rope_angles(positions, head_dim: int = 128, base: float = 10000.0) -> np.ndarray:
    pos = np.asarray(positions, dtype=np.float64)
    i = np.arange(head_dim // 2, dtype=np.float64)
    inv = base ** (-2.0 * i / head_dim)
    return pos[:, None] * inv[None, :]                   # [T, D/2]


def rope_f64(x, positions, base: float = 10000.0) -> np.ndarray:
    """x: [T, H, D] float64 -> rotated [T, H, D]."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    ang = rope_angles(positions, d, base)[:, None, :]     # [T, 1, D/2]
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., : d // 2], x[..., d // 2:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def swiglu_f64(g, u) -> np.ndarray:
    g = np.asarray(g, dtype=np.float64)
    return g / (1.0 + np.exp(-g)) * np.asarray(u, dtype=np.float64)
