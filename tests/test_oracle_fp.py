"""Pins of the oracle's floating-point foundations (CPU only).

Cited: "Defeating nondeterminism in LLM inference", section on floating-point
non-associativity (the (0.1 + 1e20) - 1e20 example, the 3-digit decimal model,
the shuffled sum of +-{1e-10, 1e-5, 1e-2, 1}); the page "same model, same input,
different answer", section on where outputs diverge (1024 values summed as 4 x 256
vs 2 x 512).
"""
import random
from decimal import Decimal, localcontext
from fractions import Fraction

import numpy as np
import pytest

from oracle import fp
from oracle.tree import sequential_sum
from tests import _scalar_ref as S


def test_nonassociativity_example_fp64_and_fp32():
    # printed on the page: (0.1 + 1e20) - 1e20 -> 0 ; 0.1 + (1e20 - 1e20) -> 0.1
    assert (0.1 + 1e20) - 1e20 == 0.0
    assert 0.1 + (1e20 - 1e20) == 0.1
    a, b = np.float32(0.1), np.float32(1e20)
    assert (a + b) - b == np.float32(0.0)
    assert a + (b - b) == np.float32(0.1)


def test_three_digit_decimal_model():
    # page: 1230 + 23.4 keeps 3 digits -> 1.25e3 ; 123 + 456 -> 579
    with localcontext() as ctx:
        ctx.prec = 3
        assert Decimal(1230) + Decimal("23.4") == Decimal("1.25E+3")
        assert Decimal(123) + Decimal(456) == Decimal(579)


def test_shuffled_sum_properties():
    """The page prints '102 unique results' with extremes +-8.3267e-17 for seed 42 and
    10 000 shuffles.  That count does not reproduce with CPython's left-to-right sum
    (parity unpinned for the literal count); the properties it illustrates are pinned:
    a fixed order gives one result, shuffled orders give several, all bounded by the
    largest rounding error of the big terms."""
    vals = [1e-10, 1e-5, 1e-2, 1]
    vals = vals + [-v for v in vals]
    random.seed(42)
    res = set()
    for _ in range(10000):
        random.shuffle(vals)
        s = 0.0
        for v in vals:                 # emulated sequential fp64 add
            s = s + v
        assert s == sum(vals)          # equals the library routine on the same order
        res.add(s)
    assert len(res) >= 2
    assert max(abs(r) for r in res) <= 2.0 ** -52
    fixed = sorted(vals)
    assert len({sum(fixed) for _ in range(100)}) == 1


def test_block_shape_changes_sum():
    # 1024 values as 4 x 256 blocks vs 2 x 512 blocks: differ for some inputs,
    # agree exactly on small integers (every partial sum exact).
    differ = 0
    for seed in range(20):
        x = np.random.default_rng(seed).standard_normal(1024).astype(np.float32)
        b4 = sequential_sum(np.stack([sequential_sum(x.reshape(4, 256))]))[0]
        b2 = sequential_sum(np.stack([sequential_sum(x.reshape(2, 512))]))[0]
        differ += int(b4 != b2)
    assert differ > 0
    xi = np.random.default_rng(0).integers(-100, 100, 1024).astype(np.float32)
    b4 = sequential_sum(np.stack([sequential_sum(xi.reshape(4, 256))]))[0]
    b2 = sequential_sum(np.stack([sequential_sum(xi.reshape(2, 512))]))[0]
    assert b4 == b2 == np.float32(xi.astype(np.int64).sum())


def test_f32_to_bf16_matches_torch():
    rng = np.random.default_rng(7)
    bits = rng.integers(0, 2 ** 32, 2_000_000, dtype=np.uint64).astype(np.uint32)
    special = np.array([0, 0x80000000, 0x7F800000, 0xFF800000, 0x3F808000, 0x3F818000,
                        0x3F807FFF, 0x7F7FFFFF, 0x00000001, 0x00008000, 0x00018000], dtype=np.uint32)
    bits = np.concatenate([bits, special])
    x = bits.view(np.float32)
    ours = fp.f32_to_bf16(x)
    ref = S.bf16_rne_torch(x)
    fin = ~np.isnan(x)
    assert np.array_equal(ours[fin], ref[fin])
    assert np.all(np.isnan(fp.bf16_to_f32(ours[~fin])))


def _bf16_from_fraction(q):
    """Independent single rounding of a rational to 8 significant bits (normal range)."""
    if q == 0:
        return 0.0
    sgn = -1 if q < 0 else 1
    a = abs(q)
    e = 0
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    unit = Fraction(2) ** (e - 7)
    n, rem = divmod(a, unit)
    if rem > unit / 2 or (rem == unit / 2 and n % 2 == 1):
        n += 1
    return sgn * float(n * unit)


def test_f64_to_bf16_single_rounding():
    rng = np.random.default_rng(3)
    x = rng.standard_normal(3000) * np.exp2(rng.integers(-60, 60, 3000))
    # values just beside bf16 ties, where rounding through fp32 first would go wrong
    ties = np.array([1.0 + 2 ** -8 + 2 ** -30, 1.0 + 2 ** -8 - 2 ** -30, 1.0 + 3 * 2 ** -8,
                     -(1.0 + 2 ** -8 + 2 ** -40)])
    x = np.concatenate([x, ties])
    got = fp.bf16_to_f64(fp.f64_to_bf16(x))
    exp = np.array([_bf16_from_fraction(Fraction(float(v))) for v in x])
    assert np.array_equal(got, exp)
    assert fp.bf16_to_f64(fp.f64_to_bf16(np.array([1.0 + 2 ** -8 + 2 ** -30])))[0] == 1.0 + 2 ** -7


def test_f32_from_fraction():
    for q in [Fraction(1, 3), Fraction(2, 3), Fraction(1, 6), Fraction(-5, 7), Fraction(1, 5040)]:
        assert fp.f32_from_fraction(q) == np.float32(float(q))   # fp64 -> fp32 is innocuous here
    assert fp.f32_from_fraction(Fraction(1) + Fraction(1, 2 ** 24)) == np.float32(1.0)
    assert fp.f32_from_fraction(Fraction(1) + Fraction(3, 2 ** 24)) == np.float32(1.0 + 2 ** -22)


def test_ulp_bf16():
    assert fp.ulp_bf16(1.0) == 2 ** -7
    assert fp.ulp_bf16(1.999) == 2 ** -7
    assert fp.ulp_bf16(2.0) == 2 ** -6
    assert fp.ulp_bf16(0.75) == 2 ** -8
