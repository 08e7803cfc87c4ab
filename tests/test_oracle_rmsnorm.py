"""Pins of the RMSNorm oracle (CPU only).

Cited: "Defeating nondeterminism in LLM inference", section "batch-invariant RMSNorm"
(y = x * rsqrt(mean(x**2)) * weight; one fixed reduction order per row whatever the
batch size).
"""
import json
import math
import os

import numpy as np

from oracle import fp
from oracle.rmsnorm import rmsnorm_tree, rmsnorm_f64
from oracle.tree import tree_sum, sequential_sum, lane_partials, lanes_for
from synth import normal_bf16, rmsnorm_linear_inputs
from tests import _scalar_ref as S

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _bits(vals):
    return fp.f32_to_bf16(np.asarray(vals, dtype=np.float32))


def test_tree_layout():
    assert lanes_for(512, 8) == 64 and lanes_for(4096, 8) == 256 and lanes_for(32000, 4) == 256
    assert lanes_for(10, 8) == 2 and lanes_for(1, 4) == 1


def test_golden_order_example():
    g = json.load(open(os.path.join(GOLD, "rmsnorm_tree_example.json")))
    x = np.zeros((1, g["D"]), dtype=np.float32)
    x[0, 0] = g["nonzero"]["0"]
    x[0, 1:16] = g["nonzero"]["1-15"]
    sq = x * x
    assert tree_sum(sq, 8)[0] == np.float32(g["tree_sum"])
    assert sequential_sum(sq)[0] == np.float32(g["sequential_sum"])
    assert tree_sum(sq, 8)[0] / np.float32(g["D"]) == np.float32(g["mean"])


def test_tree_sum_matches_scalar_lane_replay():
    rng = np.random.default_rng(11)
    for n, w in [(512, 8), (4096, 8), (1000, 4), (32000, 4), (200, 8), (77, 4), (2600, 8)]:
        v = (rng.standard_normal(n) * np.exp2(rng.integers(-20, 20, n))).astype(np.float32)
        v = np.abs(v) if w == 8 else v
        ours = tree_sum(v[None, :], w)[0]
        ref = S.tree_sum([float(t) for t in v], w)
        assert ours == np.float32(ref), (n, w)


def test_rmsnorm_matches_scalar_replay():
    x, gamma, _ = rmsnorm_linear_inputs(4, 512, 512)
    for d, eps in [(512, 1e-6)]:
        y = rmsnorm_tree(x, gamma, eps)
        xf, gf = fp.bf16_to_f32(x), fp.bf16_to_f32(gamma)
        for i in range(x.shape[0]):
            ref = S.bf16_rne_torch(S.rmsnorm_row([float(t) for t in xf[i]], [float(t) for t in gf], eps))
            assert np.array_equal(y[i], ref)
    x2 = normal_bf16((3, 4096), 0.0, 1.0, 99, 0)
    g2 = normal_bf16((4096,), 1.0, 0.02, 99, 1)
    y2 = rmsnorm_tree(x2, g2, 1e-5)
    xf, gf = fp.bf16_to_f32(x2), fp.bf16_to_f32(g2)
    for i in range(3):
        ref = S.bf16_rne_torch(S.rmsnorm_row([float(t) for t in xf[i]], [float(t) for t in gf], 1e-5))
        assert np.array_equal(y2[i], ref)


def test_integer_rows_independent_of_tree():
    # small integers: every partial sum of squares is exact, so any order gives these bits
    rng = np.random.default_rng(5)
    xi = rng.integers(-20, 21, (6, 4096)).astype(np.float32)
    g = np.ones(4096, dtype=np.float32)
    y = rmsnorm_tree(_bits(xi), _bits(g), 1e-5)
    for i in range(6):
        ssum = float(np.sum(xi[i].astype(np.int64) ** 2))
        mean = S.r32(ssum / 4096)
        r = S.r32(1.0 / S.r32(math.sqrt(S.r32(mean + S.r32(1e-5)))))
        ref = S.bf16_rne_torch([S.r32(S.r32(float(t) * r) * 1.0) for t in xi[i]])
        assert np.array_equal(y[i], ref)


def test_special_rows():
    d = 512
    zero = np.zeros((1, d), dtype=np.uint16)
    g = _bits(np.ones(d))
    y = rmsnorm_tree(zero, g, 1e-6)
    assert np.all(fp.bf16_to_f32(y) == 0.0)
    ones = _bits(np.ones((1, d)))
    y = rmsnorm_tree(ones, g, 1e-6)
    assert np.all(y == 0x3F80)             # bf16(1/sqrt(fl(1 + 1e-6))) = 1.0


def test_close_to_fp64_definition():
    x, gamma, _ = rmsnorm_linear_inputs(32, 512, 512)
    y = fp.bf16_to_f64(rmsnorm_tree(x, gamma, 1e-6))
    ref = rmsnorm_f64(x, gamma, 1e-6)
    assert np.all(np.abs(y - ref) <= fp.ulp_bf16(ref))


def test_order_sensitivity_is_real():
    # replacing the tree by a left-to-right sum changes some rows: the replay is not vacuous
    x = normal_bf16((256, 4096), 0.0, 1.0, 98, 0)
    xf = fp.bf16_to_f32(x)
    sq = xf * xf
    assert np.any(tree_sum(sq, 8) != sequential_sum(sq))
    assert lane_partials(sq, 8).shape == (256, 256)
