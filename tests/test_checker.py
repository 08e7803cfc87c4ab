"""The output checkers reject wrong answers (CPU only).

Cited: the page on verifying GPU programs before deployment: checkers that miss about
one wrong program in six, and a softmax checked at 0.01 while its outputs average
2.5e-6 so that all zeros pass; thresholds must follow the output scale, with
independent absolute, relative, range and NaN/Inf checks.
"""
import numpy as np

from oracle import fp
from oracle.check import bf16_within_1ulp, f32_within_rel, bits_equal
from oracle.gemm import gemm_f64
from synth import gemm_inputs


def _case():
    a, b = gemm_inputs(64, 256, 512, cfg=920)
    return gemm_f64(a, b)


def test_exact_answer_passes_and_wrong_answers_fail():
    ref = _case()
    good = fp.f64_to_bf16(ref)
    assert bf16_within_1ulp(good, ref)["ok"]
    assert not bf16_within_1ulp(np.zeros_like(good), ref)["ok"]
    assert not bf16_within_1ulp(np.roll(good, 1, axis=0), ref)["ok"]
    assert not bf16_within_1ulp(good.T.copy().reshape(ref.shape[1], -1)[: ref.shape[0]], ref)["ok"] \
        if ref.shape[0] == ref.shape[1] else True
    sq = ref[:, :64]
    assert not bf16_within_1ulp(fp.f64_to_bf16(sq.T), sq)["ok"]
    bad = good.copy(); bad[3, 7] = 0x7FC0
    assert not bf16_within_1ulp(bad, ref)["ok"]
    two_ulps = fp.f64_to_bf16(ref * (1 + 2 ** -6))
    assert not bf16_within_1ulp(two_ulps, ref)["ok"]
    assert not bf16_within_1ulp(good[:, :-1], ref)["ok"]


def test_tolerance_far_below_output_scale():
    ref = _case()
    floor = np.sqrt(np.mean(ref ** 2, axis=1)) / 64
    tol = fp.ulp_bf16(np.maximum(np.abs(ref), floor[:, None]))
    assert np.median(tol / np.abs(ref).mean()) < 0.01


def test_fp32_checker_and_softmax_scale():
    # a 400 000-wide softmax: outputs ~2.5e-6; all zeros must fail
    rng = np.random.default_rng(0)
    x = rng.standard_normal((1, 400_000))
    p = np.exp(x - x.max()); p /= p.sum()
    assert f32_within_rel(p.astype(np.float32), p)["ok"]
    assert not f32_within_rel(np.zeros_like(p), p)["ok"]
    assert not f32_within_rel(np.full_like(p, np.nan), p)["ok"]


def test_bits_equal():
    a = np.arange(10, dtype=np.float32)
    b = a.copy(); b[3] = -0.0 if a[3] == 0 else a[3] + 1
    assert bits_equal(a, a.copy())["ok"] and not bits_equal(a, b)["ok"]
    z = np.float32([0.0]); nz = np.float32([-0.0])
    assert not bits_equal(z, nz)["ok"]


def test_swiglu_interval_checker():
    from oracle.check import swiglu_interval_within
    from oracle.layer import swiglu_f64
    rng = np.random.default_rng(1)
    g = rng.standard_normal((4, 512)) * 1.5
    u = rng.standard_normal((4, 512)) * 1.5
    # the exact composition: rounded gate/up, SwiGLU, one rounding
    gb, ub = fp.bf16_to_f64(fp.f64_to_bf16(g)), fp.bf16_to_f64(fp.f64_to_bf16(u))
    good = fp.f64_to_bf16(swiglu_f64(gb, ub))
    assert swiglu_interval_within(good, g, u)["ok"]
    # gate values one ulp off their rounding (allowed to the projection) still pass
    g1 = fp.bf16_to_f64(fp.f64_to_bf16(gb + fp.ulp_bf16(gb)))
    assert swiglu_interval_within(fp.f64_to_bf16(swiglu_f64(g1, ub)), g, u)["ok"]
    # swapped gate and up, zeros, a missing silu, 4 ulps off, a NaN fail
    assert not swiglu_interval_within(fp.f64_to_bf16(swiglu_f64(ub, gb)), g, u)["ok"]
    assert not swiglu_interval_within(np.zeros_like(good), g, u)["ok"]
    assert not swiglu_interval_within(fp.f64_to_bf16(gb * ub), g, u)["ok"]
    off = fp.bf16_to_f64(good) * (1 + 2 ** -5)
    assert not swiglu_interval_within(fp.f64_to_bf16(off), g, u)["ok"]
    bad = good.copy(); bad[1, 3] = 0x7FC0
    assert not swiglu_interval_within(bad, g, u)["ok"]


def test_drift_reports():
    from oracle.check import drift_report, logit_drift_report
    rng = np.random.default_rng(2)
    ref = rng.standard_normal((1, 4096)) * 2.5
    r = drift_report(fp.f64_to_bf16(ref), ref)
    assert r["frac_exact"] == 1.0 and r["frac_within_1ulp"] == 1.0 and r["max_over_rms"] < 2 ** -6
    r = drift_report(fp.f64_to_bf16(-ref), ref)
    assert r["frac_exact"] < 0.01 and r["mean_over_rms"] > 1.0
    lg = rng.standard_normal((3, 100))
    got = lg.copy()
    got[1, np.argmax(lg[1])] -= 10.0                 # row 1 loses its top token
    rep = logit_drift_report(got, lg, k=5)
    assert rep["token_agreement"] == 2 / 3 and rep["topk_agreement"] == 2 / 3
    assert rep["max_abs"] == 10.0 and rep["rows"] == 3
    top2 = np.sort(lg, axis=1)[:, -2:]
    assert rep["min_margin"] == float((top2[:, 1] - top2[:, 0]).min())
