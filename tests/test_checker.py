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


def test_composed_drift_rejects_gross_errors():
    from oracle.check import composed_drift
    rng = np.random.default_rng(1)
    ref = rng.standard_normal((1, 4096)) * 2.5
    good = fp.f64_to_bf16(ref)
    assert composed_drift(good, ref)["ok"]
    # an ulp of noise on a third of the elements still passes
    noisy = fp.bf16_to_f64(good).copy()
    sel = rng.random((1, 4096)) < 0.33
    noisy[sel] += fp.ulp_bf16(noisy[sel]) * rng.choice([-1, 1], int(sel.sum()))
    assert composed_drift(fp.f64_to_bf16(noisy), ref)["ok"]
    # a missing residual term, a sign flip or zeros fail
    assert not composed_drift(fp.f64_to_bf16(ref * 0.7), ref)["ok"]
    assert not composed_drift(fp.f64_to_bf16(-ref), ref)["ok"]
    assert not composed_drift(np.zeros_like(good), ref)["ok"]
    wrong = ref.copy(); wrong[0, :300] += 0.5
    assert not composed_drift(fp.f64_to_bf16(wrong), ref)["ok"]
