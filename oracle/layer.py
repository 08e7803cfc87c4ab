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


# ---------------------------------------------------------------------------------
# Decoder layer and model, fp64 arithmetic with bf16 storage between operations.
#
# The bf16 model stores every activation in bf16, so the definition of its forward pass
# includes one round-to-nearest-even at each of those points; inside each operation the
# oracle computes in fp64 (RMSNorm by its bit-exact tree definition).  A GPU result can
# still differ where an intermediate lies within rounding error of a bf16 tie, so the
# composed outputs are graded with a tolerance derived from that (tests say how).
def _r(x):
    from .fp import bf16_to_f64, f64_to_bf16
    return bf16_to_f64(f64_to_bf16(x))


def decoder_layer_ref(h_bits, w, positions, prior_k, prior_v, eps=1e-5, base=10000.0,
                      n_q_heads=32, n_kv_heads=8, head_dim=128):
    """h_bits [T, D] bf16 bits; w: dict of bf16 bit arrays (Linear [out, in]); token t sits
    at positions[t] with prior_k[t], prior_v[t] [positions[t], Hkv, hd] bf16 bits of its
    earlier keys/values.  Returns (out fp64 [T, D] before the final rounding, dict)."""
    from .attention import attention_rows_f64
    from .fp import bf16_to_f64, f64_to_bf16
    from .gemm import gemm_f64
    from .rmsnorm import rmsnorm_tree
    h = bf16_to_f64(h_bits)
    T = h.shape[0]
    x = rmsnorm_tree(h_bits, w["attn_norm"], eps)
    qkv = _r(gemm_f64(x, w["wqkv"], "nk"))
    qn, kn = n_q_heads * head_dim, n_kv_heads * head_dim
    q = qkv[:, :qn].reshape(T, n_q_heads, head_dim)
    k = qkv[:, qn:qn + kn].reshape(T, n_kv_heads, head_dim)
    v = qkv[:, qn + kn:].reshape(T, n_kv_heads, head_dim)
    qr = f64_to_bf16(rope_f64(q, positions, base))
    kr = f64_to_bf16(rope_f64(k, positions, base))
    vb = f64_to_bf16(v)
    a = np.zeros((T, n_q_heads, head_dim))
    for t in range(T):
        K = np.concatenate([prior_k[t], kr[t:t + 1]])
        V = np.concatenate([prior_v[t], vb[t:t + 1]])
        a[t] = attention_rows_f64(qr[t:t + 1], K, V, [int(positions[t])])[0]
    a = _r(a).reshape(T, qn)
    o = _r(gemm_f64(f64_to_bf16(a), w["wo"], "nk"))
    h2 = _r(h + o)
    x2 = rmsnorm_tree(f64_to_bf16(h2), w["ffn_norm"], eps)
    gu = _r(gemm_f64(x2, w["wgate_up"], "nk"))
    F = gu.shape[1] // 2
    m = _r(swiglu_f64(gu[:, :F], gu[:, F:]))
    dn = _r(gemm_f64(f64_to_bf16(m), w["wdown"], "nk"))
    return h2 + dn, dict(x=x, q=qr, k=kr, v=vb, attn=a, h2=h2, mlp=m, dn=dn)


def model_ref_logits(prompt, forced, weights, eps=1e-5, base=10000.0, n_q_heads=32,
                     n_kv_heads=8, head_dim=128, fp32_variant=False):
    """Logits (fp64) after the prompt and after each teacher-forced token, for a model
    given as weights = dict(embed, layers=[layer dicts], final_norm, lm_head) of bf16 bit
    arrays.  One sequence; the bf16 model (fp32_variant=False) stores activations in
    bf16 as in decoder_layer_ref."""
    from .attention import attention_rows_f64
    from .fp import bf16_to_f64, f64_to_bf16
    from .gemm import gemm_f64
    from .rmsnorm import rmsnorm_tree
    if fp32_variant:
        raise NotImplementedError("the oracle replays the bf16 model only")
    L = len(weights["layers"])
    ctx_k = [np.zeros((0, n_kv_heads, head_dim), np.uint16) for _ in range(L)]
    ctx_v = [np.zeros((0, n_kv_heads, head_dim), np.uint16) for _ in range(L)]
    out = []
    seqs = [list(prompt)] + [[t] for t in forced]
    pos0 = 0
    for toks in seqs:
        T = len(toks)
        h_bits = weights["embed"][np.asarray(toks)]
        positions = np.arange(pos0, pos0 + T)
        for li, w in enumerate(weights["layers"]):
            h = bf16_to_f64(h_bits)
            x = rmsnorm_tree(h_bits, w["attn_norm"], eps)
            qkv = _r(gemm_f64(x, w["wqkv"], "nk"))
            qn, kn = n_q_heads * head_dim, n_kv_heads * head_dim
            q = qkv[:, :qn].reshape(T, n_q_heads, head_dim)
            k = qkv[:, qn:qn + kn].reshape(T, n_kv_heads, head_dim)
            v = qkv[:, qn + kn:].reshape(T, n_kv_heads, head_dim)
            qr = f64_to_bf16(rope_f64(q, positions, base))
            ctx_k[li] = np.concatenate([ctx_k[li], f64_to_bf16(rope_f64(k, positions, base))])
            ctx_v[li] = np.concatenate([ctx_v[li], f64_to_bf16(v)])
            a = attention_rows_f64(qr, ctx_k[li], ctx_v[li], positions)
            a = _r(a).reshape(T, qn)
            o = _r(gemm_f64(f64_to_bf16(a), w["wo"], "nk"))
            h2 = _r(h + o)
            x2 = rmsnorm_tree(f64_to_bf16(h2), w["ffn_norm"], eps)
            gu = _r(gemm_f64(x2, w["wgate_up"], "nk"))
            F = gu.shape[1] // 2
            m = _r(swiglu_f64(gu[:, :F], gu[:, F:]))
            dn = _r(gemm_f64(f64_to_bf16(m), w["wdown"], "nk"))
            h_bits = f64_to_bf16(h2 + dn)
        xf = rmsnorm_tree(h_bits[-1:], weights["final_norm"], eps)
        out.append(gemm_f64(xf, weights["lm_head"], "nk")[0])
        pos0 += T
    return np.stack(out)
