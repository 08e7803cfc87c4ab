"""bi_add_rmsnorm_gemm and bi_add_rmsnorm_gemm_swiglu (residual add + RMSNorm + projection in
one launch) on the GPU: the sum and the product equal, bit for bit, bi_add_rmsnorm followed by
bi_gemm / bi_gemm_swiglu, which the RMSNorm and GEMM tests grade against the oracle -- at every
row count the fused calls take, on both weight layouts, bf16 and fp32 products, with a partial
last K step, fewer tree lanes than 256 (K < 2048), the largest K (4096; 8192 is refused) and
ragged N; and one case against the oracle directly.

Cited: "Defeating nondeterminism in LLM inference", section on batch-invariant RMSNorm (each
row keeps its fixed reduction order whatever kernel computes it) and section on batch-invariant
matrix multiplication (the same instruction sequence per output element).
"""
import numpy as np
import pytest
import torch

from oracle import fp
from oracle.check import bf16_within_1ulp
from oracle.gemm import gemm_f64
from oracle.rmsnorm import rmsnorm_tree
from synth import normal_bf16
from tests._gpu import bf16, bits, same_bits, say

pytestmark = pytest.mark.gpu

EPS = 1e-5


def _rows(k, seed):
    a = normal_bf16((4, k), 0.0, 1.0, 70, seed)
    b = normal_bf16((4, k), 0.0, 0.5, 70, seed + 1)
    g = normal_bf16((k,), 1.0, 0.02, 70, seed + 2)
    return a, b, g


@pytest.mark.parametrize("n,k", [(6144, 4096), (1000, 1032), (4096, 8192), (48, 2048), (272, 1024), (512, 3000)])
def test_fused_norm_gemm_equals_unfused(lib, n, k):
    say("add_rmsnorm_gemm", n, k)
    from invariant_amd import BI_B_NK, BI_B_TILED, BIError
    a, b, g = _rows(k, n + k)
    A, B, G = bf16(a), bf16(b), bf16(g)
    W = bf16(normal_bf16((n, k), 0.0, 0.02, 71, n))
    Wt = lib.bi_pack_b(W)
    for m in (1, 2, 3, 4):
        if k > 4096:   # the staged rows must fit 32 KB of LDS
            with pytest.raises(BIError):
                lib.bi_add_rmsnorm_gemm(A[:m], B[:m], G, EPS, W)
            continue
        s_ref, y_ref = lib.bi_add_rmsnorm(A[:m], B[:m], G, EPS)
        for od in (torch.bfloat16, torch.float32):
            c_ref = lib.bi_gemm(y_ref, W, out_dtype=od)
            for layout, w in ((BI_B_NK, W), (BI_B_TILED, Wt)):
                s, c = lib.bi_add_rmsnorm_gemm(A[:m], B[:m], G, EPS, w, w_layout=layout, n=n, out_dtype=od)
                assert same_bits(s, s_ref), (m, od, layout)
                assert same_bits(c, c_ref), (m, od, layout)


@pytest.mark.parametrize("f,k", [(14336, 4096), (1024, 1024), (3008, 1032)])
def test_fused_norm_gemm_swiglu_equals_unfused(lib, f, k):
    say("add_rmsnorm_gemm_swiglu", f, k)
    from invariant_amd import BI_B_NK, BI_B_TILED, interleave_gate_up
    a, b, g = _rows(k, f + k)
    A, B, G = bf16(a), bf16(b), bf16(g)
    Wi = interleave_gate_up(bf16(normal_bf16((2 * f, k), 0.0, 0.02, 72, f)))
    Wt = lib.bi_pack_b(Wi)
    for m in (1, 2, 3, 4):
        s_ref, y_ref = lib.bi_add_rmsnorm(A[:m], B[:m], G, EPS)
        o_ref = lib.bi_gemm_swiglu(y_ref, Wi)
        for layout, w in ((BI_B_NK, Wi), (BI_B_TILED, Wt)):
            s, o = lib.bi_add_rmsnorm_gemm_swiglu(A[:m], B[:m], G, EPS, w, w_layout=layout)
            assert same_bits(s, s_ref), (m, layout)
            assert same_bits(o, o_ref), (m, layout)


def test_fused_norm_gemm_vs_oracle(lib):
    # the sum is one rounding of the exact sum; the product is within 1 bf16 ulp of the fp64
    # product of the oracle's tree-replayed RMSNorm of that sum
    n, k = 512, 4096
    a, b, g = _rows(k, 9)
    w = normal_bf16((n, k), 0.0, 0.02, 73, 0)
    s, c = lib.bi_add_rmsnorm_gemm(bf16(a[:3]), bf16(b[:3]), bf16(g), EPS, bf16(w))
    s_ref = fp.f64_to_bf16(fp.bf16_to_f64(a[:3]) + fp.bf16_to_f64(b[:3]))
    assert np.array_equal(bits(s), s_ref)
    y = rmsnorm_tree(s_ref, g, EPS)
    r = bf16_within_1ulp(bits(c), gemm_f64(y, w, "nk"))
    assert r["ok"], r


def test_sum_overlapping_inputs_is_refused(lib):
    # the sum is written by one workgroup while the others still read a and b
    from invariant_amd import BIError
    a, b, g = _rows(1024, 5)
    A, B = bf16(a), bf16(b)
    W = bf16(normal_bf16((64, 1024), 0.0, 0.02, 74, 0))
    with pytest.raises(BIError):
        lib.bi_add_rmsnorm_gemm(A, B, bf16(g), EPS, W, sum_out=A)
