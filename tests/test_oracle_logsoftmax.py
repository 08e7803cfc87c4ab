"""Pins of the log-softmax / argmax oracle and its EXP / LOG (CPU only).

Cited: greedy decoding = always the most likely token ("Defeating nondeterminism in
LLM inference", introduction; "same LLM, different GPU", greedy decoding and token
probabilities from normalised scores); near-tie argmax flip ("same model, same input,
different answer", section on sampling).
"""
import math

import numpy as np

from oracle import fp
from oracle.logsoftmax import EXP, LOG, K, logsoftmax_argmax, logsoftmax_f64, argmax_first
from tests import _scalar_ref as S


def test_exp_accuracy_and_specials():
    rng = np.random.default_rng(0)
    d = np.concatenate([-rng.random(3_000_000).astype(np.float32) * np.float32(86.5),
                        -np.abs(rng.standard_normal(500_000)).astype(np.float32),
                        np.float32([-0.0, 0.0, -1e-30, -1e-45, -86.0, -0.34657359, -0.3465736])])
    e = EXP(d).astype(np.float64)
    t = np.exp(d.astype(np.float64))
    assert np.max(np.abs(e - t) / fp.ulp_f32(t)) <= 2.0
    assert EXP(np.float32([0.0]))[0] == 1.0 and EXP(np.float32([-0.0]))[0] == 1.0
    assert np.isnan(EXP(np.float32([np.nan]))[0])
    assert EXP(np.float32([-np.inf]))[0] == 0.0
    # flush below 2^-125 (k < -125) to +0, values above stay normal
    far = -np.linspace(87.5, 200, 1000).astype(np.float32)
    assert np.all(EXP(far) == 0.0)
    near = -np.linspace(0, 86.5, 100000).astype(np.float32)
    assert np.all(EXP(near) >= np.float32(2.0 ** -126))


def test_log_accuracy_and_specials():
    rng = np.random.default_rng(1)
    s = np.concatenate([(1 + rng.random(2_000_000) * 2 ** 20).astype(np.float32),
                        np.float32([1.0, 1.5, 2.0, 32000.0, 1.4142135, 1.4142137, 2.0 ** 24])])
    got = LOG(s).astype(np.float64)
    t = np.log(s.astype(np.float64))
    assert np.max(np.abs(got - t) / fp.ulp_f32(np.maximum(t, 1e-30))) <= 2.0
    assert LOG(np.float32([1.0]))[0] == 0.0
    assert np.isnan(LOG(np.float32([np.nan]))[0]) and LOG(np.float32([np.inf]))[0] == np.inf


def test_constants_from_their_definitions():
    assert abs(float(K["LN2_HI"]) + float(K["LN2_LO"]) - math.log(2)) < 2e-13
    assert int(np.float32(K["LN2_HI"]).view(np.uint32)) & 0xFF == 0      # 16 significant bits
    assert K["EXP_C"][0] == 1 and K["EXP_C"][2] == 0.5 and K["LOG_B"][0] == 2


def test_uniform_row():
    v = 32000
    x = np.full((2, v), 0.75, dtype=np.float32)
    lp, a = logsoftmax_argmax(x)
    assert np.all(a == 0)
    assert np.all(lp == -LOG(np.float32([v]))[0])
    assert abs(float(lp[0, 0]) + math.log(v)) <= 2 * float(fp.ulp_f32(math.log(v)))


def test_one_hot_row():
    v = 1000
    x = np.zeros((1, v), dtype=np.float32)
    x[0, 17] = 150.0
    lp, a = logsoftmax_argmax(x)
    assert a[0] == 17 and lp[0, 17] == 0.0
    assert np.all(lp[0, np.arange(v) != 17] == np.float32(-150.0))


def test_argmax_ties_nan_near_tie():
    x = np.zeros((4, 16), dtype=np.float32)
    x[0, 5] = x[0, 9] = 2.0                         # tie -> lowest index
    x[1, 3] = np.float32(3.4819); x[1, 11] = np.float32(3.4821)   # near tie
    x[2, 6] = np.nan; x[2, 2] = np.nan              # NaN counts as max, first one
    x[3, :] = -0.0; x[3, 4] = 0.0                   # -0 == +0 -> index 0
    a = argmax_first(x)
    assert list(a) == [5, 11, 2, 0]
    # brute force
    for r in range(4):
        best = 0
        for j in range(16):
            xj, xb = x[r, j], x[r, best]
            if (np.isnan(xj) and not np.isnan(xb)) or (not np.isnan(xb) and xj > xb):
                best = j
        assert a[r] == best


def test_sum_matches_scalar_replay_and_probabilities_sum_to_one():
    rng = np.random.default_rng(4)
    x = (rng.standard_normal((3, 32000)) * 2).astype(np.float32)
    lp, a = logsoftmax_argmax(x)
    for r in range(3):
        m = x[r, a[r]]
        d = x[r] - m
        e = EXP(d)
        s = S.tree_sum([float(t) for t in e], 4)
        L = LOG(np.float32([s]))[0]
        assert np.array_equal(lp[r], d - L)
    ref = logsoftmax_f64(x)
    assert np.max(np.abs(lp - ref)) < 1e-5
    assert abs(np.exp(lp.astype(np.float64)).sum(axis=1) - 1).max() < 1e-5
    for v in (1000, 37, 1, 4099):
        xs = (rng.standard_normal((1, v))).astype(np.float32)
        lp, a = logsoftmax_argmax(xs)
        e = EXP(xs[0] - xs[0, a[0]])
        assert S.tree_sum([float(t) for t in e], 4) == float(LOG.__globals__["tree_sum"](e[None, :], 4)[0])


def test_c_replay_equals_python_oracle():
    # oracle/explog.c (used for the exhaustive GPU sweeps) is the Python oracle's EXP and LOG
    # bit for bit: on a stride through every float of each domain, on random values, and on
    # the special values
    from oracle import explog_c
    from oracle.logsoftmax import EXP, LOG
    bits = np.arange(0x80000000, 0xC2D00001, 97, dtype=np.uint64).astype(np.uint32)
    x = np.concatenate([bits.view(np.float32),
                        np.float32([0.0, -0.0, -np.inf, np.nan, -87.33654, -103.97208])])
    assert np.array_equal(explog_c.EXP(x).view(np.uint32), EXP(x).view(np.uint32))
    s = np.arange(0x3F800000, 0x47000001, 13, dtype=np.uint32).view(np.float32)
    s = np.concatenate([s, np.float32([1.0, 32768.0, np.inf, np.nan, 1.4142135])])
    assert np.array_equal(explog_c.LOG(s).view(np.uint32), LOG(s).view(np.uint32))
    first = 0xC2000000
    assert np.array_equal(explog_c.exp_bits(first, 1000).view(np.uint32),
                          EXP((np.arange(1000, dtype=np.uint32) + np.uint32(first)).view(np.float32)).view(np.uint32))
