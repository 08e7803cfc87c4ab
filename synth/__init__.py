"""Seeded synthetic inputs shared by the oracle tests, the GPU parity tests and the bench.

This module only draws random numbers and lays them out; it holds none of the
arithmetic of the path (no normalisation, products, softmax or reductions).
Every tensor is drawn from ``numpy.random.Generator(PCG64([cfg, tensor, layer]))``
so a (config id, tensor id, layer id) triple names its values on any host.

Values that the path consumes as bf16 are returned as ``uint16`` bit patterns.
The float32 -> bf16 step uses torch's CPU conversion (round to nearest even),
which is part of drawing the input, not of the method.

The second argument of every N(mean, sd) below is the standard deviation.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "rng", "normal_bf16", "bf16_to_f32", "uniform_ints", "ragged_lengths",
    "rmsnorm_linear_inputs", "gemm_inputs", "attention_case", "paged_layout",
    "layer_weights", "model_dims", "MISTRAL",
]

MISTRAL = dict(hidden=4096, n_q_heads=32, n_kv_heads=8, head_dim=128, ffn=14336,
               vocab=32000, n_layers=32, rms_eps=1e-5, rope_base=10000.0)


def model_dims():
    return dict(MISTRAL)


def rng(cfg: int, tensor: int, layer: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64([int(cfg), int(tensor), int(layer)]))


def _f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 values (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def normal_bf16(shape, mean: float, sd: float, cfg: int, tensor: int, layer: int = 0) -> np.ndarray:
    g = rng(cfg, tensor, layer)
    x = g.standard_normal(size=shape, dtype=np.float32)
    if sd != 1.0:
        x *= np.float32(sd)
    if mean != 0.0:
        x += np.float32(mean)
    return _f32_to_bf16_bits(x)


def normal_f32(shape, mean: float, sd: float, cfg: int, tensor: int, layer: int = 0) -> np.ndarray:
    g = rng(cfg, tensor, layer)
    x = g.standard_normal(size=shape, dtype=np.float32)
    return (x * np.float32(sd) + np.float32(mean)).astype(np.float32)


def uniform_ints(n: int, lo: int, hi: int, cfg: int, tensor: int, layer: int = 0) -> np.ndarray:
    """n integers uniform in [lo, hi] (both ends included)."""
    return rng(cfg, tensor, layer).integers(lo, hi, size=n, endpoint=True).astype(np.int64)


def ragged_lengths(n: int, lo: int, hi: int, cfg: int, tensor: int) -> np.ndarray:
    return uniform_ints(n, lo, hi, cfg, tensor)


# ---------------------------------------------------------------- workloads
def rmsnorm_linear_inputs(max_m: int = 32, d: int = 512, n: int = 512, cfg: int = 1):
    """RMSNorm + linear batch sweep: x ~ N(0,1) [max_m, d], gamma ~ N(1, 0.02) [d],
    W ~ N(0, 1/d) as an [n, d] Linear weight (the product is x_hat @ W^T)."""
    x = normal_bf16((max_m, d), 0.0, 1.0, cfg, 0)
    gamma = normal_bf16((d,), 1.0, 0.02, cfg, 1)
    w = normal_bf16((n, d), 0.0, 1.0 / d, cfg, 2)
    return x, gamma, w


def gemm_inputs(m: int, n: int, k: int, cfg: int = 2, sd: float = 1.0):
    """A ~ N(0, sd) [m, k]; B ~ N(0, sd) drawn as [k, n] (torch.mm orientation)."""
    a = normal_bf16((m, k), 0.0, sd, cfg, 0)
    b = normal_bf16((k, n), 0.0, sd, cfg, 1)
    return a, b


def paged_layout(seq_lens, page_size: int, cfg: int, tensor: int, extra_pages: int = 0):
    """Assign every sequence ceil(L/page) physical pages drawn as a random permutation
    of the page pool, so that logical order never matches physical order.
    Returns (block_table int32 [B, max_pages], n_pages)."""
    seq_lens = np.asarray(seq_lens, dtype=np.int64)
    pages_per = (seq_lens + page_size - 1) // page_size
    total = int(pages_per.sum()) + extra_pages
    perm = rng(cfg, tensor).permutation(total).astype(np.int32)
    max_pages = int(max(1, pages_per.max(initial=1)))
    bt = np.full((len(seq_lens), max_pages), -1, dtype=np.int32)
    off = 0
    for b, p in enumerate(pages_per):
        bt[b, :p] = perm[off:off + p]
        off += p
    return bt, total


def attention_case(seq_lens, q_lens, n_q_heads=32, n_kv_heads=8, head_dim=128,
                   cfg: int = 4, salt: int = 0, sd: float = 1.0):
    """Logical per-sequence K/V and the new tokens' q for one attention call.

    Sequence b holds seq_lens[b] tokens after the call; its last q_lens[b] tokens are
    new.  K/V of a sequence are drawn in one stream (a longer draw extends a shorter
    one) and q is drawn per absolute position, so the same token has the same inputs
    whether it arrives in a prefill (all tokens new) or a decode (one token new).
    Returns k[b], v[b]: [L, Hkv, D] and q[b]: [q_b, Hq, D] as bf16 bits."""
    seq_lens = [int(s) for s in seq_lens]
    q_lens = [int(q) for q in q_lens]
    ks, vs, qs = [], [], []
    for b, (L, ql) in enumerate(zip(seq_lens, q_lens)):
        ks.append(normal_bf16((L, n_kv_heads, head_dim), 0.0, sd, cfg, 100 + 3 * b, salt))
        vs.append(normal_bf16((L, n_kv_heads, head_dim), 0.0, sd, cfg, 101 + 3 * b, salt))
        if ql:
            qs.append(np.stack([normal_bf16((n_q_heads, head_dim), 0.0, sd, cfg, 102 + 3 * b,
                                            (salt << 20) + p) for p in range(L - ql, L)]))
        else:
            qs.append(np.zeros((0, n_q_heads, head_dim), dtype=np.uint16))
    return dict(seq_lens=seq_lens, q_lens=q_lens, k=ks, v=vs, q=qs)


def layer_weights(hidden=4096, n_q_heads=32, n_kv_heads=8, head_dim=128, ffn=14336,
                  cfg: int = 3, layer: int = 0, sd: float = 0.02):
    """Mistral-shaped decoder-layer weights as Linear [out, in] bf16 bit patterns.
    Linear matrices ~ N(0, sd); RMSNorm gammas ~ N(1, 0.02)."""
    qkv_out = (n_q_heads + 2 * n_kv_heads) * head_dim
    return dict(
        attn_norm=normal_bf16((hidden,), 1.0, 0.02, cfg, 10, layer),
        wqkv=normal_bf16((qkv_out, hidden), 0.0, sd, cfg, 11, layer),
        wo=normal_bf16((hidden, n_q_heads * head_dim), 0.0, sd, cfg, 12, layer),
        ffn_norm=normal_bf16((hidden,), 1.0, 0.02, cfg, 13, layer),
        wgate_up=normal_bf16((2 * ffn, hidden), 0.0, sd, cfg, 14, layer),
        wdown=normal_bf16((hidden, ffn), 0.0, sd, cfg, 15, layer),
    )
