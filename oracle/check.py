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


def swiglu_interval_within(got_bits, g_ref, u_ref, axis=-1) -> dict:
    """Output of a fused gate/up projection + SwiGLU (bf16) against the fp64 gate and up
    values g_ref, u_ref of the projection.  The projection's own bar lets each stored gate
    value lie anywhere within tol_g = ulp_bf16(max(|g|, rms_row(g)/64)) of bf16_rne(g) (and
    likewise u); swiglu(g, u) = silu(g) u is evaluated over that box (corners, plus silu's
    minimum at g* = -1.27846... when the box holds it) and the result must lie within one
    ulp of the output scale of [bf16_rne(min), bf16_rne(max)]."""
    got = bf16_to_f64(np.asarray(got_bits, dtype=np.uint16))
    g = np.asarray(g_ref, dtype=np.float64)
    u = np.asarray(u_ref, dtype=np.float64)
    if got.shape != g.shape or g.shape != u.shape:
        return dict(ok=False, reason="shape")
    if not np.all(np.isfinite(got)):
        return dict(ok=False, reason="non-finite output")

    def box(x):
        r = bf16_to_f64(f64_to_bf16(x))
        t = ulp_bf16(np.maximum(np.abs(x), _row_floor(x, axis=axis)))
        return r - t, r + t

    def sw(a, b):
        return a / (1.0 + np.exp(-a)) * b

    glo, ghi = box(g)
    ulo, uhi = box(u)
    cands = [sw(a, b) for a in (glo, ghi) for b in (ulo, uhi)]
    gstar = -1.2784645427610738        # silu'(g*) = 0: 1 + g* (1 - silu(g*)/g*) = 0
    inside = (glo <= gstar) & (gstar <= ghi)
    for b in (ulo, uhi):
        cands.append(np.where(inside, sw(gstar, b), cands[0]))
    lo = np.minimum.reduce(cands)
    hi = np.maximum.reduce(cands)
    ref = sw(g, u)
    tol = ulp_bf16(np.maximum(np.maximum(np.abs(lo), np.abs(hi)), _row_floor(ref, axis=axis)))
    lo_r = bf16_to_f64(f64_to_bf16(lo)) - tol
    hi_r = bf16_to_f64(f64_to_bf16(hi)) + tol
    bad = (got < lo_r) | (got > hi_r)
    return dict(ok=not bool(bad.any()), n_bad=int(bad.sum()),
                frac_exact=float(np.mean(got == bf16_to_f64(f64_to_bf16(ref)))))


def drift_report(got_bits, ref64, axis=-1) -> dict:
    """How far a composed bf16 computation (a whole layer) sits from an fp64 chain:
    max and mean |error| over the row rms, the fraction within one own-magnitude ulp and
    the fraction equal to the rounded reference.  Reported, not a verdict: two correct bf16
    chains round their stored intermediates differently, and wide later sums add those
    ulps up; the composition is graded op by op."""
    got = bf16_to_f64(np.asarray(got_bits, dtype=np.uint16))
    ref64 = np.asarray(ref64, dtype=np.float64)
    rms = np.sqrt(np.mean(ref64 ** 2, axis=axis, keepdims=True))
    err = np.abs(got - ref64)
    rb = bf16_to_f64(f64_to_bf16(ref64))
    within1 = np.abs(got - rb) <= ulp_bf16(np.maximum(np.abs(ref64), 1e-30))
    return dict(max_over_rms=float((err / rms).max()), mean_over_rms=float((err / rms).mean()),
                frac_within_1ulp=float(within1.mean()), frac_exact=float(np.mean(got == rb)))


def logit_drift_report(got, ref, k: int = 5) -> dict:
    """Mismatch of logits [rows, V] against a reference, in the metric families of the
    cross-vendor abstract (logit difference, top-K consistency, token agreement) and the
    top-1/top-2 margin that decides greedy flips (page on different answers, sampling):
    max and mean |dlogit| (absolute and over the reference row rms), the fraction of rows
    whose top-k sets agree, of rows whose argmax agrees, and the reference margins."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    d = np.abs(got - ref)
    rms = np.sqrt(np.mean(ref ** 2, axis=1, keepdims=True))
    tk_g = np.sort(np.argsort(-got, axis=1, kind="stable")[:, :k], axis=1)
    tk_r = np.sort(np.argsort(-ref, axis=1, kind="stable")[:, :k], axis=1)
    top2 = np.sort(ref, axis=1)[:, -2:]
    margin = top2[:, 1] - top2[:, 0]
    return dict(rows=int(ref.shape[0]), max_abs=float(d.max()), mean_abs=float(d.mean()),
                max_over_rms=float((d / rms).max()), mean_over_rms=float((d / rms).mean()),
                topk=k, topk_agreement=float(np.mean(np.all(tk_g == tk_r, axis=1))),
                token_agreement=float(np.mean(np.argmax(got, 1) == np.argmax(ref, 1))),
                min_margin=float(margin.min()), median_margin=float(np.median(margin)),
                max_err_over_min_margin=float(d.max() / max(margin.min(), 1e-300)))
