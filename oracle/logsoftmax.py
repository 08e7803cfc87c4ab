"""Log-softmax and greedy argmax oracle, with the EXP and LOG that are part of the
contract.

Sources: greedy decoding picks the highest-probability token ("same LLM, different
GPU", sections on greedy decoding and token probabilities from normalised scores);
"Defeating nondeterminism in LLM inference" (temperature 0 = always the most likely
token; the reduction order must be fixed); the page "same model, same input,
different answer" (a near tie such as 3.4821 vs 3.4819 flips an argmax).

Per row x (fp32 logits):
  a   = lowest index attaining the maximum (a NaN counts as the maximum; -0 == +0)
  m   = x[a]
  d_i = x_i - m                        (fp32)
  s   = tree_sum(EXP(d_i)), 4-element vectors (16-byte fp32 loads)
  L   = LOG(s)
  logprob_i = d_i - L                  (fp32)

The maximum with lowest-index ties is a selection under a total order, so it is the
same for every reduction tree; only the sum needs the tree replay.

EXP and LOG are written from published methods, in fp32 with every multiply and add
rounded separately (no fused multiply-add), so that both sides can replay them:
  EXP(d), d <= 0 or NaN  -- Cody & Waite (1980) argument reduction:
      k = rint(d * LOG2E);  r = (d - k*LN2_HI) - k*LN2_LO;
      exp(r) by the degree-7 Taylor polynomial in Horner form, coefficients 1/n!
      rounded to fp32;  result = p * 2^k built from exponent bits.
      k < -125 (the result would be below 2^-125) returns +0; NaN returns NaN.
  LOG(s), s >= 1, +inf or NaN  -- reduction to f in [sqrt(1/2), sqrt(2)) and the
      atanh series log f = 2(z + z^3/3 + ... + z^15/15), z = (f-1)/(f+1)
      (J.-M. Muller, Elementary Functions, ch. on table-free range reduction):
      result = e*LN2_HI + (e*LN2_LO + z*q(z^2)).
Constants are derived here from exact rationals (ln 2 and sqrt 2 from 60-digit
decimal arithmetic), never taken from a vendor library.
"""
from __future__ import annotations

import math
from decimal import Decimal, localcontext
from fractions import Fraction

import numpy as np

from .fp import f32_from_fraction
from .tree import tree_sum


def _constants():
    with localcontext() as ctx:
        ctx.prec = 60
        ln2 = Fraction(Decimal(2).ln())
        sqrt2 = Fraction(Decimal(2).sqrt())
    # ln 2 rounded to 16 significant bits: k * LN2_HI is exact for |k| < 2^8
    hi = Fraction(round(ln2 * 2 ** 16), 2 ** 16)
    return dict(
        LOG2E=f32_from_fraction(1 / ln2),
        LN2_HI=np.float32(float(hi)),
        LN2_LO=f32_from_fraction(ln2 - hi),
        SQRT2=f32_from_fraction(sqrt2),
        EXP_C=[f32_from_fraction(Fraction(1, math.factorial(n))) for n in range(8)],
        LOG_B=[f32_from_fraction(Fraction(2, 2 * i + 1)) for i in range(8)],
    )


K = _constants()
F32 = np.float32


def EXP(d) -> np.ndarray:
    d = np.asarray(d, dtype=np.float32)
    nan = np.isnan(d)
    t = d * K["LOG2E"]
    k = np.rint(t)
    with np.errstate(invalid="ignore"):
        live = (~nan) & (k >= F32(-125.0))
    kk = np.where(live, k, F32(0.0)).astype(np.float32)
    r = d - kk * K["LN2_HI"]
    r = r - kk * K["LN2_LO"]
    c = K["EXP_C"]
    p = np.full(d.shape, c[7], dtype=np.float32)
    for n in range(6, -1, -1):
        p = p * r + c[n]
    scale = ((kk.astype(np.int32) + np.int32(127)) << np.int32(23)).astype(np.int32).view(np.float32)
    res = p * scale
    out = np.where(live, res, F32(0.0)).astype(np.float32)
    return np.where(nan, d, out).astype(np.float32)


def LOG(s) -> np.ndarray:
    s = np.asarray(s, dtype=np.float32)
    special = ~np.isfinite(s)
    ss = np.where(special, F32(1.0), s).astype(np.float32)
    bits = ss.view(np.uint32)
    e = (bits >> np.uint32(23)).astype(np.int32) - np.int32(127)
    f = ((bits & np.uint32(0x7FFFFF)) | np.uint32(0x3F800000)).view(np.float32)
    big = f > K["SQRT2"]
    f = np.where(big, f * F32(0.5), f).astype(np.float32)
    e = np.where(big, e + 1, e)
    z = (f - F32(1.0)) / (f + F32(1.0))
    w = z * z
    b = K["LOG_B"]
    q = np.full(s.shape, b[7], dtype=np.float32)
    for i in range(6, -1, -1):
        q = q * w + b[i]
    lf = z * q
    ef = e.astype(np.float32)
    res = ef * K["LN2_HI"] + (ef * K["LN2_LO"] + lf)
    return np.where(special, s, res).astype(np.float32)


def argmax_first(x) -> np.ndarray:
    """Lowest index of the maximum per row (NaN counts as the maximum)."""
    return np.argmax(np.asarray(x, dtype=np.float32), axis=-1).astype(np.int32)


def logsoftmax_argmax(x):
    """x: float32 [M, V] -> (logprobs float32 [M, V], argmax int32 [M])."""
    x = np.asarray(x, dtype=np.float32)
    a = argmax_first(x)
    m = x[np.arange(x.shape[0]), a]
    with np.errstate(invalid="ignore"):
        d = x - m[:, None]
    e = EXP(d)
    s = tree_sum(e, 4)
    L = LOG(s)
    with np.errstate(invalid="ignore"):
        lp = d - L[:, None]
    return lp.astype(np.float32), a


def logsoftmax_f64(x) -> np.ndarray:
    x = np.asarray(x, dtype=np.float64)
    m = x.max(axis=-1, keepdims=True)
    return (x - m) - np.log(np.sum(np.exp(x - m), axis=-1, keepdims=True))
