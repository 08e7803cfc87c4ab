"""Causal GQA attention oracle over logical (unpaged) sequences, in fp64.

Source: "Defeating nondeterminism in LLM inference", section "batch-invariant
attention": attention reduces over the feature and the sequence dimensions; the
K/V cache and page table are updated before the attention kernel runs, so a query
token reduces over the same keys whether it arrives in a prefill or in a decode.

For sequence b with L_b tokens after the call, its last q_b tokens are the queries;
token at absolute position p of query head h attends to keys 0..p of kv head
h // (Hq / Hkv):

    o[p, h] = sum_j softmax_j(q[p,h] . k[j, g] / sqrt(D)) v[j, g],  j = 0..p.

The split into fixed 256-token chunks and the merge of chunk partials is the GPU's
way of computing this sum; mathematically it is the same quantity, so the oracle is
the plain definition and the GPU result is graded within 1 bf16 ulp of it at the
scale rms(o[p, h]) / 64.
"""
from __future__ import annotations

import numpy as np

from .fp import bf16_to_f64


def attention_rows_f64(q_bits, k_bits, v_bits, positions, n_kv_heads=None) -> np.ndarray:
    """q_bits [T, Hq, D] for the query tokens at absolute ``positions`` (length T);
    k_bits, v_bits [L, Hkv, D] logical keys/values of the sequence.
    Returns o [T, Hq, D] float64."""
    q = bf16_to_f64(q_bits)
    k = bf16_to_f64(k_bits)
    v = bf16_to_f64(v_bits)
    t, hq, d = q.shape
    hkv = k.shape[1]
    g = hq // hkv
    out = np.zeros((t, hq, d), dtype=np.float64)
    scale = 1.0 / np.sqrt(d)
    for i, p in enumerate(np.asarray(positions, dtype=np.int64)):
        kk = k[: p + 1]                                   # [p+1, Hkv, D]
        vv = v[: p + 1]
        for h in range(hq):
            s = kk[:, h // g, :] @ q[i, h] * scale        # [p+1]
            w = np.exp(s - s.max())
            out[i, h] = (w @ vv[:, h // g, :]) / w.sum()
    return out


def attention_case_f64(case, which=None) -> list:
    """All new tokens of every sequence in an ``synth.attention_case`` dict.
    ``which``: optional {b: list of new-token indices} to compute only some rows."""
    outs = []
    for b, (L, ql) in enumerate(zip(case["seq_lens"], case["q_lens"])):
        idx = list(range(ql)) if which is None else list(which.get(b, []))
        pos = [L - ql + i for i in idx]
        qb = case["q"][b][idx] if idx else case["q"][b][:0]
        outs.append(attention_rows_f64(qb, case["k"][b][:L], case["v"][b][:L], pos))
    return outs
