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


def attention_values_f64(q, k, v, positions, block: int = 512) -> np.ndarray:
    """The definition above on float64 values: q [T, Hq, D] (queries at absolute
    ``positions``), k, v [L, Hkv, D] (keys/values of positions 0..L-1).  Per kv head, the
    scores of its query heads and a block of queries are one matrix product and the
    weighted sum another (library products as steps; the arithmetic is the plain fp64
    softmax-weighted sum).  Returns o [T, Hq, D] float64."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    pos = np.asarray(positions, dtype=np.int64)
    t, hq, d = q.shape
    hkv = k.shape[1]
    g = hq // hkv
    out = np.zeros((t, hq, d), dtype=np.float64)
    if t == 0:
        return out
    scale = 1.0 / np.sqrt(d)
    for b0 in range(0, t, block):
        b1 = min(t, b0 + block)
        pb = pos[b0:b1]
        n = int(pb.max()) + 1                                # keys any query here can see
        row_pos = np.repeat(pb, g)                           # rows: (query, head of the group)
        mask = np.arange(n)[None, :] <= row_pos[:, None]
        for h in range(hkv):
            kh = k[:n, h, :]                                 # [n, D]
            vh = v[:n, h, :]
            qh = q[b0:b1, h * g:(h + 1) * g, :].reshape(-1, d)    # [(b1 - b0) G, D]
            s = np.where(mask, (qh @ kh.T) * scale, -np.inf)
            w = np.exp(s - s.max(axis=1, keepdims=True))
            o = (w @ vh) / w.sum(axis=1, keepdims=True)
            out[b0:b1, h * g:(h + 1) * g, :] = o.reshape(b1 - b0, g, d)
    return out


def attention_rows_f64(q_bits, k_bits, v_bits, positions, n_kv_heads=None) -> np.ndarray:
    """q_bits [T, Hq, D] for the query tokens at absolute ``positions`` (length T);
    k_bits, v_bits [L, Hkv, D] logical keys/values of the sequence (bf16 bits).
    Returns o [T, Hq, D] float64."""
    return attention_values_f64(bf16_to_f64(q_bits), bf16_to_f64(k_bits), bf16_to_f64(v_bits),
                                positions)


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
