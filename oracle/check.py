"""Output checkers with tolerances stated per output scale.

The page on verifying GPU programs before deployment (section on an over-loose
tolerance) shows a softmax whose outputs average 2.5e-6 checked at 0.01: an
all-zero answer passes.  Every band here is therefore tied to the scale of the
expected output, per row (GEMM) or per (token, head) vector (attention):

  floor_i      = rms_j(ref_ij) / 64
  bf16 output  : |got - bf16_rne(ref)| <= ulp_bf16(max(|ref_ij|, floor_i))
  fp32 output  : |got - ref| <= 1e-3 * max(|ref_ij|, floor_i)

plus shape, NaN/Inf agreement and bit equality checks.  Each returns a report dict;
``ok`` is the verdict.
"""
from __future__ import annotations

import numpy as np

from .fp import bf16_to_f64, f64_to_bf16, ulp_bf16

FLOOR_DIV = 64.0


def _row_floor(ref: np.ndarray, axis=-1) -> np.ndarray:
    rms = np.sqrt(np.mean(np.square(ref), axis=axis, keepdims=True))
    return rms / FLOOR_DIV


def bf16_within_1ulp(got_bits: np.ndarray, ref64: np.ndarray, axis=-1) -> dict:
    """bf16 result vs fp64 reference: within one bf16 ulp of bf16_rne(ref) at the
    magnitude max(|ref|, rms(row)/64)."""
    got_bits = np.asarray(got_bits, dtype=np.uint16)
    ref64 = np.asarray(ref64, dtype=np.float64)
    if got_bits.shape != ref64.shape:
        return dict(ok=False, reason=f"shape {got_bits.shape} != {ref64.shape}")
    got = bf16_to_f64(got_bits)
    if not np.all(np.isfinite(ref64)):
        same_nan = np.array_equal(np.isnan(got), np.isnan(ref64))
        fin = np.isfinite(ref64)
        if not same_nan or not np.array_equal(got[~fin & ~np.isnan(ref64)], ref64[~fin & ~np.isnan(ref64)]):
            return dict(ok=False, reason="non-finite mismatch")
    else:
        fin = np.ones(ref64.shape, dtype=bool)
        if not np.all(np.isfinite(got)):
            return dict(ok=False, reason="non-finite output")
    rb = bf16_to_f64(f64_to_bf16(ref64))
    floor = _row_floor(np.where(fin, ref64, 0.0), axis=axis)
    tol = ulp_bf16(np.maximum(np.abs(ref64), floor))
    err = np.abs(got - rb)
    err = np.where(fin, err, 0.0)
    bad = err > tol
    ulps = np.where(fin, err / tol, 0.0)
    return dict(ok=not bool(bad.any()), n_bad=int(bad.sum()), max_ulps=float(ulps.max(initial=0.0)),
                frac_exact=float(np.mean(err == 0.0)) if err.size else 1.0)


def f32_within_rel(got: np.ndarray, ref64: np.ndarray, rel: float = 1e-3, axis=-1) -> dict:
    got = np.asarray(got, dtype=np.float64)
    ref64 = np.asarray(ref64, dtype=np.float64)
    if got.shape != ref64.shape:
        return dict(ok=False, reason=f"shape {got.shape} != {ref64.shape}")
    if not np.all(np.isfinite(got)):
        return dict(ok=False, reason="non-finite output")
    floor = _row_floor(ref64, axis=axis)
    tol = rel * np.maximum(np.abs(ref64), floor)
    err = np.abs(got - ref64)
    bad = err > tol
    return dict(ok=not bool(bad.any()), n_bad=int(bad.sum()),
                max_rel=float((err / np.maximum(np.abs(ref64), floor)).max(initial=0.0)))


def bits_equal(a: np.ndarray, b: np.ndarray) -> dict:
    a = np.ascontiguousarray(a)
    b = np.ascontiguousarray(b)
    if a.shape != b.shape or a.dtype.itemsize != b.dtype.itemsize:
        return dict(ok=False, reason=f"shape/dtype {a.shape}/{a.dtype} vs {b.shape}/{b.dtype}")
    ua = a.view(np.uint8).reshape(a.shape + (-1,))
    ub = b.view(np.uint8).reshape(b.shape + (-1,))
    diff = np.any(ua != ub, axis=-1)
    return dict(ok=not bool(diff.any()), n_diff=int(diff.sum()))


def residual_sum_within(got_bits, ref64, terms, n_ulp: float = 2.0, axis=-1) -> dict:
    """A bf16 output that ends in a sum out = t_1 + t_2 + ... of stored bf16 terms (a
    residual add).  Two correct evaluations may round each stored term differently (by
    one ulp of that term), and the sum can cancel, so the band is set by the terms:
        |got - bf16_rne(ref)| <= n_ulp * ulp_bf16(max_k |t_k|) + ulp_bf16(max(|ref|, floor))
    with floor = rms(ref row) / 64 as in bf16_within_1ulp."""
    got = bf16_to_f64(np.asarray(got_bits, dtype=np.uint16))
    ref64 = np.asarray(ref64, dtype=np.float64)
    if got.shape != ref64.shape:
        return dict(ok=False, reason=f"shape {got.shape} != {ref64.shape}")
    if not np.all(np.isfinite(got)):
        return dict(ok=False, reason="non-finite output")
    big = np.max(np.stack([np.abs(np.asarray(t, dtype=np.float64)) for t in terms]), axis=0)
    floor = _row_floor(ref64, axis=axis)
    tol = n_ulp * ulp_bf16(big) + ulp_bf16(np.maximum(np.abs(ref64), floor))
    err = np.abs(got - bf16_to_f64(f64_to_bf16(ref64)))
    bad = err > tol
    return dict(ok=not bool(bad.any()), n_bad=int(bad.sum()), max_of_tol=float((err / tol).max()),
                frac_exact=float(np.mean(err == 0.0)))


def composed_drift(got_bits, ref64, axis=-1) -> dict:
    """Drift of a composed bf16 computation (a whole decoder layer) from its oracle chain.

    Two correct bf16 chains round their stored intermediates differently at about one
    element in several hundred per operation; wide later sums (a 4096- or 14336-long dot
    product) add those one-ulp differences up, so after a layer about a third of the
    outputs differ by an ulp or two and the largest differences reach a few percent of
    the row rms.  A wrong weight, rotation or mask moves outputs by the order of the rms
    itself, so the gate is:
        max |err| <= rms / 8,  mean |err| <= rms / 256,  >= 2/3 within one own-ulp."""
    got = bf16_to_f64(np.asarray(got_bits, dtype=np.uint16))
    ref64 = np.asarray(ref64, dtype=np.float64)
    if got.shape != ref64.shape or not np.all(np.isfinite(got)):
        return dict(ok=False, reason="shape or non-finite")
    rms = np.sqrt(np.mean(ref64 ** 2, axis=axis, keepdims=True))
    err = np.abs(got - ref64)
    rb = bf16_to_f64(f64_to_bf16(ref64))
    within1 = np.abs(got - rb) <= ulp_bf16(np.maximum(np.abs(ref64), 1e-30))
    mx, mean = float((err / rms).max()), float((err / rms).mean())
    f1 = float(within1.mean())
    return dict(ok=mx <= 1 / 8 and mean <= 1 / 256 and f1 >= 2 / 3, max_over_rms=mx, mean_over_rms=mean,
                frac_within_1ulp=f1, frac_exact=float(np.mean(got == rb)))
