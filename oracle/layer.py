"""Decoder-layer and model oracle (Mistral-7B-shaped composition).

TEST INFRASTRUCTURE (see oracle/__init__.py): only tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py use it; the HIP path never does.

The pointwise steps around the three reductions ("Defeating nondeterminism in LLM
inference", section on making kernels batch-invariant: pointwise operations are
batch-invariant as long as every element runs the same code):

  RoPE    : rotate-half pairing (i, i + D/2), angle p * base^(-2i/D), i < D/2
  SwiGLU  : silu(g) * u = g / (1 + exp(-g)) * u, g the first half of the gate/up output
  residual: h + f(h)

Readings (the pages name these steps but print no formula): rotate-half pairing, base
10000, angles in fp64.

Layer (pre-norm, as in Mistral-7B):
  x  = rmsnorm(h);  q, k, v = rope(split(x Wqkv^T));  a = attention(q | cache + k, v)
  h2 = h + a Wo^T;  x2 = rmsnorm(h2);  out = h2 + swiglu(x2 Wgu^T) Wd^T

Every operation computes in fp64 (RMSNorm by its bit-exact tree replay) and its result is
rounded once to the type the model STORES it in.  Storage points:
  bf16 model      every activation bf16; logits fp32 (graded against fp64).
  FP32/MLP-BF16   ("cross-vendor mismatch" abstract: upcast to FP32 except the MLPs, which
  variant         stay BF16) the residual stream h, the attention-side norm output x, the
                  fused projection qkv, the attention output a, the projection o, h2 and
                  the layer output are fp32 (weights stay bf16 and enter exactly); q is
                  fp32 (Spec.q_dtype; bf16 on request); k and v are bf16, the type of the KV cache
                  (storage, as the weights are); the MLP -- its norm output x2, the gate/up
                  values, the SwiGLU output and the down projection -- is bf16; the final
                  norm is fp32.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .attention import attention_values_f64
from .fp import bf16_to_f64, f64_to_bf16
from .gemm import gemm_f64
from .rmsnorm import rmsnorm_tree


@dataclass(frozen=True)
class Spec:
    n_q_heads: int = 32
    n_kv_heads: int = 8
    head_dim: int = 128
    eps: float = 1e-5
    base: float = 10000.0
    variant: bool = False      # the FP32/MLP-BF16 variant
    q_dtype: str = "f32"       # storage of q in the variant ("f32" or "bf16"); bf16 model: bf16

    @property
    def act(self) -> str:
        return "f32" if self.variant else "bf16"


# ---------------------------------------------------------------------------- storage
def store(x, dtype: str) -> np.ndarray:
    """fp64 values -> the fp64 values of their stored type (one rounding)."""
    x = np.asarray(x, dtype=np.float64)
    if dtype == "bf16":
        return bf16_to_f64(f64_to_bf16(x))
    if dtype == "f32":
        return x.astype(np.float32).astype(np.float64)
    raise ValueError(dtype)


def _as_input(x64, dtype: str):
    """Stored fp64 values -> what rmsnorm_tree / gemm_f64 take for that type."""
    return f64_to_bf16(x64) if dtype == "bf16" else np.asarray(x64, dtype=np.float32)


# ---------------------------------------------------------------------------- operations
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


def split_qkv(qkv, spec: Spec):
    """[T, (Hq + 2 Hkv) D] -> q [T, Hq, D], k [T, Hkv, D], v [T, Hkv, D] (no arithmetic)."""
    t = qkv.shape[0]
    qn, kn = spec.n_q_heads * spec.head_dim, spec.n_kv_heads * spec.head_dim
    return (qkv[:, :qn].reshape(t, spec.n_q_heads, spec.head_dim),
            qkv[:, qn:qn + kn].reshape(t, spec.n_kv_heads, spec.head_dim),
            qkv[:, qn + kn:].reshape(t, spec.n_kv_heads, spec.head_dim))


def op_rmsnorm(h64, gamma_bits, eps, in_dtype: str, out_dtype: str) -> np.ndarray:
    """RMSNorm of stored values (tree replay, bit-exact); returns the stored output values."""
    y = rmsnorm_tree(_as_input(h64, in_dtype), gamma_bits, eps, in_dtype, out_dtype)
    return bf16_to_f64(y) if out_dtype == "bf16" else np.asarray(y, dtype=np.float64)


def op_gemm(a64, w_bits, a_dtype: str) -> np.ndarray:
    """a . W^T in fp64 for a Linear weight W [out, in]; a holds stored values of a_dtype."""
    return gemm_f64(_as_input(a64, a_dtype), w_bits, "nk", a_dtype=a_dtype)


def op_rope_qkv(qkv64, positions, spec: Spec):
    """Split the fused projection (stored values) and rotate q and k: fp64 (q, k, v)."""
    q, k, v = split_qkv(np.asarray(qkv64, dtype=np.float64), spec)
    return rope_f64(q, positions, spec.base), rope_f64(k, positions, spec.base), v


def op_attention(q64, k64, v64, positions) -> np.ndarray:
    return attention_values_f64(q64, k64, v64, positions)


# ---------------------------------------------------------------------------- layer
def _layer(h, w, positions, spec: Spec, attend):
    """One layer on stored residual values h [T, hidden].  attend(q, k, v) returns the
    fp64 attention output [T, Hq, D] from the stored q and the new tokens' stored k, v.
    Returns (out, intermediates), all as stored values."""
    act = spec.act
    t = h.shape[0]
    x = op_rmsnorm(h, w["attn_norm"], spec.eps, act, act)
    qkv = store(op_gemm(x, w["wqkv"], act), act)
    q, k, v = op_rope_qkv(qkv, positions, spec)
    q = store(q, spec.q_dtype if spec.variant else "bf16")
    k, v = store(k, "bf16"), store(v, "bf16")
    a = store(attend(q, k, v), act).reshape(t, spec.n_q_heads * spec.head_dim)
    o = store(op_gemm(a, w["wo"], act), act)
    h2 = store(h + o, act)
    x2 = op_rmsnorm(h2, w["ffn_norm"], spec.eps, act, "bf16")
    gu = store(op_gemm(x2, w["wgate_up"], "bf16"), "bf16")
    f = gu.shape[1] // 2
    m = store(swiglu_f64(gu[:, :f], gu[:, f:]), "bf16")
    dn = store(op_gemm(m, w["wdown"], "bf16"), "bf16")
    out = store(h2 + dn, act)
    return out, dict(x=x, qkv=qkv, q=q, k=k, v=v, attn=a, o=o, h2=h2, x2=x2, gu=gu, mlp=m, dn=dn)


def sequence_layer_ref(h, w, pos0: int, ctx_k, ctx_v, spec: Spec):
    """T consecutive tokens of ONE sequence at positions pos0 .. pos0 + T - 1 whose keys and
    values of positions 0 .. pos0 - 1 are ctx_k, ctx_v [pos0, Hkv, D] (stored values); the
    new tokens attend to those and, causally, to each other.  h: stored values [T, hidden].
    Returns (out, intermediates); intermediates["k"], ["v"] extend the context."""
    t = h.shape[0]
    positions = np.arange(pos0, pos0 + t)

    def attend(q, k, v):
        return op_attention(q, np.concatenate([ctx_k, k]), np.concatenate([ctx_v, v]), positions)

    return _layer(h, w, positions, spec, attend)


def decoder_layer_ref(h_bits, w, positions, prior_k, prior_v, eps=1e-5, base=10000.0,
                      n_q_heads=32, n_kv_heads=8, head_dim=128):
    """Independent single-token requests (the batched-decode form): token t sits at
    positions[t] with prior_k[t], prior_v[t] [positions[t], Hkv, D] bf16 bits of its
    request's earlier keys/values.  bf16 model.  Returns (out, intermediates) as stored
    fp64 values (out holds bf16 values)."""
    spec = Spec(n_q_heads, n_kv_heads, head_dim, eps, base)
    positions = np.asarray(positions, dtype=np.int64)

    def attend(q, k, v):
        a = np.zeros((q.shape[0], n_q_heads, head_dim))
        for i in range(q.shape[0]):
            kk = np.concatenate([bf16_to_f64(prior_k[i]), k[i:i + 1]])
            vv = np.concatenate([bf16_to_f64(prior_v[i]), v[i:i + 1]])
            a[i] = op_attention(q[i:i + 1], kk, vv, positions[i:i + 1])[0]
        return a

    return _layer(bf16_to_f64(h_bits), w, positions, spec, attend)


# ---------------------------------------------------------------------------- model
def embed_ref(weights, tokens, spec: Spec) -> np.ndarray:
    """Embedding rows as stored values (a gather; exact widening for the variant)."""
    return bf16_to_f64(weights["embed"][np.asarray(tokens, dtype=np.int64)])


def head_ref(weights, h_rows, spec: Spec) -> np.ndarray:
    """Final norm (stored in the activation type) and the LM head: fp64 logits."""
    xf = op_rmsnorm(h_rows, weights["final_norm"], spec.eps, spec.act, spec.act)
    return op_gemm(xf, weights["lm_head"], spec.act)


def model_ref_forward(pieces, weights, spec: Spec, logit_rows=None, on_layer=None):
    """The model over one sequence fed in consecutive pieces of tokens (a prefill, then a
    decode step per token, or any other split), the KV context growing piece by piece.
    weights = dict(embed, layers=[layer dicts], final_norm, lm_head) of bf16 bit arrays.
    logit_rows(i, T) -> rows of piece i whose logits are wanted (default: its last row).
    on_layer(piece, layer, h_in, out, intermediates) is called after every layer.
    Returns a list with the fp64 logits [rows, V] of each piece."""
    n_layers = len(weights["layers"])
    hkv, hd = spec.n_kv_heads, spec.head_dim
    ctx_k = [np.zeros((0, hkv, hd)) for _ in range(n_layers)]
    ctx_v = [np.zeros((0, hkv, hd)) for _ in range(n_layers)]
    out = []
    pos0 = 0
    for i, toks in enumerate(pieces):
        toks = np.asarray(toks, dtype=np.int64)
        t = len(toks)
        h = embed_ref(weights, toks, spec)
        for li, w in enumerate(weights["layers"]):
            h_in = h
            h, inter = sequence_layer_ref(h, w, pos0, ctx_k[li], ctx_v[li], spec)
            ctx_k[li] = np.concatenate([ctx_k[li], inter["k"]])
            ctx_v[li] = np.concatenate([ctx_v[li], inter["v"]])
            if on_layer is not None:
                on_layer(i, li, h_in, h, inter)
        rows = [t - 1] if logit_rows is None else list(logit_rows(i, t))
        out.append(head_ref(weights, h[rows], spec))
        pos0 += t
    return out


def model_ref_logits(prompt, forced, weights, eps=1e-5, base=10000.0, n_q_heads=32,
                     n_kv_heads=8, head_dim=128, fp32_variant=False, q_dtype="f32",
                     one_pass=False):
    """Teacher-forced logits (fp64) after the prompt and after each forced token: [1 +
    len(forced), V].  By default the prompt is one piece and every forced token its own
    decode step; one_pass=True feeds prompt + forced as one piece and reads the same rows
    (causality makes the two equal)."""
    spec = Spec(n_q_heads, n_kv_heads, head_dim, eps, base, fp32_variant, q_dtype)
    prompt = [int(t) for t in prompt]
    forced = [int(t) for t in forced]
    if one_pass:
        p = len(prompt)
        lg = model_ref_forward([prompt + forced], weights, spec,
                               logit_rows=lambda i, t: range(p - 1, t))
        return lg[0]
    pieces = [prompt] + [[t] for t in forced]
    return np.concatenate(model_ref_forward(pieces, weights, spec))
