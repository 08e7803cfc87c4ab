"""Scalar, pure-Python re-derivations used only to pin the vectorised oracle.

Every fp32 operation is done in fp64 on fp32 operands and rounded once to fp32.
For one +, -, *, / or sqrt of fp32 operands this equals the correctly rounded fp32
result, because binary64 has at least 2*24 + 2 significant bits (double rounding is
then innocuous).  The code walks lanes and butterfly exchanges explicitly instead of
reshaping arrays, so it shares no indexing with the oracle.
"""
import math
from fractions import Fraction

import numpy as np


def r32(x: float) -> float:
    return float(np.float32(x))


def tree_sum(vals, width):
    n = len(vals)
    nvec = -(-n // width)
    t = max(1, min(256, nvec))
    lanes = [0.0] * t
    for v in range(nvec):                       # ascending: each lane sees its vectors in order
        lane = v % t
        for e in range(width):
            i = v * width + e
            if i < n:
                lanes[lane] = r32(lanes[lane] + vals[i])
    waves = []
    for w in range(-(-t // 64)):
        cur = [lanes[64 * w + j] if 64 * w + j < t else 0.0 for j in range(64)]
        for off in (1, 2, 4, 8, 16, 32):
            cur = [r32(cur[j] + cur[j ^ off]) for j in range(64)]
        assert all(c == cur[0] for c in cur)
        waves.append(cur[0])
    if len(waves) == 1:
        return waves[0]
    if len(waves) == 2:
        return r32(waves[0] + waves[1])
    waves = waves + [0.0] * (4 - len(waves))
    return r32(r32(waves[0] + waves[1]) + r32(waves[2] + waves[3]))


def bf16_rne_torch(vals):
    import torch
    return torch.tensor(np.asarray(vals, dtype=np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def rmsnorm_row(x_vals, g_vals, eps):
    """One row, scalar: returns float32 values before the bf16 rounding."""
    sq = [r32(x * x) for x in x_vals]
    s = tree_sum(sq, 8)
    mean = r32(s / len(x_vals))
    v = r32(mean + r32(eps))
    rt = r32(math.sqrt(v))
    r = r32(1.0 / rt)
    return [r32(r32(x * r) * g) for x, g in zip(x_vals, g_vals)]


def matmul_fraction(a, b):
    a = [[Fraction(float(x)) for x in row] for row in a]
    b = [[Fraction(float(x)) for x in row] for row in b]
    m, k, n = len(a), len(b), len(b[0])
    return [[sum(a[i][kk] * b[kk][j] for kk in range(k)) for j in range(n)] for i in range(m)]


def attention_scalar(q, k, v, p, g):
    """q [Hq, D], k/v [L, Hkv, D] python floats; positions 0..p; fp64 math.exp."""
    hq, d = len(q), len(q[0])
    out = []
    for h in range(hq):
        kv = h // g
        s = [sum(q[h][t] * k[j][kv][t] for t in range(d)) / math.sqrt(d) for j in range(p + 1)]
        mx = max(s)
        w = [math.exp(x - mx) for x in s]
        tot = sum(w)
        out.append([sum(w[j] * v[j][kv][t] for j in range(p + 1)) / tot for t in range(d)])
    return out
