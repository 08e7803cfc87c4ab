"""bi_gemm_fixed_split on the GPU: K cut into slices of a fixed length at absolute offsets
for every M, each slice bi_gemm's fp32 chain, the slices added in ascending order.

Cited: "Defeating nondeterminism in LLM inference": batch-invariant RMSNorm (last
paragraph: a strategy with enough parallelism for tiny batches is invariant when every
batch size uses it) and batch-invariant matrix multiplication (split-K for small M and N).
"""
import numpy as np
import pytest
import torch

from oracle import fp
from oracle.check import bf16_within_1ulp
from oracle.gemm import gemm_f64
from synth import gemm_inputs
from tests._gpu import bf16, bits, host, same_bits, say

pytestmark = pytest.mark.gpu


def _nk(b_kn):
    return np.ascontiguousarray(b_kn.T)


@pytest.mark.parametrize("m,n,k,ks", [(1, 512, 4096, 1024), (64, 1024, 4096, 1024),
                                      (300, 1024, 4000, 1024), (33, 600, 3000, 64),
                                      (4, 4100, 14336, 2048), (700, 300, 1000, 256)])
def test_vs_oracle(lib, m, n, k, ks):
    # few-row and LDS-staged kernels, ragged K (a short last slice), one-stage slices
    say("fixed split", m, n, k, ks)
    a, b = gemm_inputs(m, n, k, cfg=61)
    c = lib.bi_gemm_fixed_split(bf16(a), bf16(_nk(b)), ks)
    r = bf16_within_1ulp(bits(c), gemm_f64(a, b))
    assert r["ok"], r


@pytest.mark.parametrize("m,n,k,ks", [(64, 512, 2504, 1024), (5, 700, 4096, 512), (300, 256, 1088, 64)])
def test_is_slice_chains_added_in_order(lib, m, n, k, ks):
    # the definition: slice s = bi_gemm over columns [s ks, (s + 1) ks) in fp32, then
    # ((0 + slice 0) + slice 1) + .. in fp32, rounded once to bf16
    a, b = gemm_inputs(m, n, k, cfg=62)
    A, W = bf16(a), bf16(_nk(b))
    acc = np.zeros((m, n), dtype=np.float32)
    for s0 in range(0, k, ks):
        s1 = min(k, s0 + ks)
        part = lib.bi_gemm(A[:, s0:s1], W[:, s0:s1], out_dtype=torch.float32)
        acc = acc + host(part)
    got = lib.bi_gemm_fixed_split(A, W, ks, out_dtype=torch.float32)
    assert np.array_equal(host(got).view(np.uint32), acc.view(np.uint32))
    got16 = lib.bi_gemm_fixed_split(A, W, ks)
    assert np.array_equal(bits(got16), fp.f32_to_bf16(acc))


@pytest.mark.parametrize("n,k,ks", [(4096, 4096, 1024), (4096, 14336, 2048), (1000, 3000, 1024)])
def test_rows_bitwise_equal_for_every_m(lib, n, k, ks):
    # the rows of M = 1, 3, 17, .. equal the same rows of the 2048-row call under every
    # kernel configuration those M select, and rows gathered from anywhere in the batch
    full_m = 2048
    a, b = gemm_inputs(full_m, n, k, cfg=63)
    A, W = bf16(a), bf16(_nk(b))
    full = lib.bi_gemm_fixed_split(A, W, ks)
    fullf = lib.bi_gemm_fixed_split(A, W, ks, out_dtype=torch.float32)
    configs = set()
    for m in (1, 3, 17, 33, 64, 65, 128, 511, 1024):
        configs.add(lib.bi_gemm_tile(m, n, k))
        assert same_bits(lib.bi_gemm_fixed_split(A[:m], W, ks), full[:m]), (n, k, m)
        assert same_bits(lib.bi_gemm_fixed_split(A[:m], W, ks, out_dtype=torch.float32), fullf[:m]), (n, k, m)
    say("fixed split configurations", n, k, sorted(configs))
    assert len(configs) >= 3
    sel = torch.tensor([full_m - 1, 17, 1500, 300], device="cuda")
    assert same_bits(lib.bi_gemm_fixed_split(A[sel].contiguous(), W, ks), full[sel])


def test_one_slice_is_bi_gemm(lib):
    a, b = gemm_inputs(40, 512, 1024, cfg=64)
    A, W = bf16(a), bf16(_nk(b))
    ref = lib.bi_gemm(A, W)
    for ks in (1024, 2048, 1 << 20):
        assert same_bits(lib.bi_gemm_fixed_split(A, W, ks), ref)
