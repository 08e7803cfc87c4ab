"""bi_rmsnorm on the GPU: bit-exact against the tree-replaying oracle, batch-invariant.

Cited: "Defeating nondeterminism in LLM inference", section on batch-invariant RMSNorm.
"""
import numpy as np
import pytest
import torch

from oracle import fp
from oracle.rmsnorm import rmsnorm_tree
from synth import normal_bf16, rmsnorm_linear_inputs
from tests._gpu import bf16, bits, f32, host, same_bits, say

pytestmark = pytest.mark.gpu


def test_rmsnorm_512_batch_sweep_bit_exact(lib):
    x, gamma, _ = rmsnorm_linear_inputs(32, 512, 512)
    ref = rmsnorm_tree(x, gamma, 1e-6)
    X, G = bf16(x), bf16(gamma)
    row0 = None
    for m in range(1, 33):
        y = lib.bi_rmsnorm(X[:m], G, 1e-6)
        torch.cuda.synchronize()
        assert np.array_equal(bits(y), ref[:m]), m
        row0 = y[0].clone() if row0 is None else row0
        assert same_bits(y[0], row0)


@pytest.mark.parametrize("m,d,eps", [(1, 4096, 1e-5), (7, 4096, 1e-5), (300, 4096, 1e-5),
                                     (5, 14336, 1e-5), (3, 1000, 1e-6), (4, 12, 1e-6),
                                     (2, 9000, 1e-5), (9, 100, 0.5), (3, 1, 1e-6), (2, 8, 1e-6)])
def test_shapes_bit_exact(lib, m, d, eps):
    say("rmsnorm", m, d)
    x = normal_bf16((m, d), 0.0, 1.0, 21, d)
    g = normal_bf16((d,), 1.0, 0.02, 21, d + 1)
    y = lib.bi_rmsnorm(bf16(x), bf16(g), eps)
    assert np.array_equal(bits(y), rmsnorm_tree(x, g, eps))


def test_strided_and_fp32_variants(lib):
    d = 4096
    x = normal_bf16((6, d + 64), 0.0, 3.0, 22, 0)
    g = normal_bf16((d,), 1.0, 0.02, 22, 1)
    X = bf16(x)[:, :d]                                   # row stride d + 64
    y = lib.bi_rmsnorm(X, bf16(g), 1e-5)
    assert np.array_equal(bits(y), rmsnorm_tree(np.ascontiguousarray(x[:, :d]), g, 1e-5))
    xf = (np.random.default_rng(0).standard_normal((5, d)) * 2).astype(np.float32)
    yf = lib.bi_rmsnorm(f32(xf), bf16(g), 1e-5, out_dtype=torch.float32)
    assert np.array_equal(host(yf).view(np.uint32),
                          rmsnorm_tree(xf, g, 1e-5, in_dtype="f32", out_dtype="f32").view(np.uint32))
    yb = lib.bi_rmsnorm(f32(xf), bf16(g), 1e-5)
    assert np.array_equal(bits(yb), rmsnorm_tree(xf, g, 1e-5, in_dtype="f32"))
    yfb = lib.bi_rmsnorm(bf16(x[:, :d].copy()), bf16(g), 1e-5, out_dtype=torch.float32)
    assert np.array_equal(host(yfb).view(np.uint32),
                          rmsnorm_tree(np.ascontiguousarray(x[:, :d]), g, 1e-5, out_dtype="f32").view(np.uint32))


def test_special_rows(lib):
    d = 512
    x = np.zeros((4, d), dtype=np.float32)
    x[1] = 1.0
    x[2, 7] = np.nan
    x[3, 0] = 4096.0; x[3, 1:16] = 1.0                  # order-sensitive row
    xb = fp.f32_to_bf16(x)
    g = fp.f32_to_bf16(np.ones(d, dtype=np.float32))
    y = bits(lib.bi_rmsnorm(bf16(xb), bf16(g), 1e-6))
    ref = rmsnorm_tree(xb, g, 1e-6)
    fin = ~np.isnan(fp.bf16_to_f32(ref))
    assert np.array_equal(y[fin], ref[fin])
    assert np.all(np.isnan(fp.bf16_to_f32(y[2])))
    assert np.all(y[1] == 0x3F80)


def test_large_m_sampled_and_invariant(lib):
    m, d = 65536, 4096
    gen = torch.Generator(device="cuda").manual_seed(5)
    X = torch.randn((m, d), generator=gen, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    g = normal_bf16((d,), 1.0, 0.02, 23, 0)
    G = bf16(g)
    Y = lib.bi_rmsnorm(X, G, 1e-5)
    rows = np.array([0, 1, 777, 32768, 65535])
    xs = bits(X[torch.from_numpy(rows).cuda()])
    assert np.array_equal(bits(Y[torch.from_numpy(rows).cuda()]), rmsnorm_tree(xs, g, 1e-5))
    # the same rows alone, and the batch permuted: bitwise equal
    for r in rows:
        assert same_bits(lib.bi_rmsnorm(X[r:r + 1], G, 1e-5)[0], Y[r])
    perm = torch.randperm(4096, generator=torch.Generator().manual_seed(1)).cuda()
    Yp = lib.bi_rmsnorm(X[:4096][perm].contiguous(), G, 1e-5)
    assert same_bits(Yp, Y[:4096][perm])


def test_repeat_determinism(lib):
    x = normal_bf16((64, 4096), 0.0, 1.0, 24, 0)
    g = normal_bf16((4096,), 1.0, 0.02, 24, 1)
    X, G = bf16(x), bf16(g)
    ref = lib.bi_rmsnorm(X, G, 1e-5)
    for _ in range(200):
        assert same_bits(lib.bi_rmsnorm(X, G, 1e-5), ref)


@pytest.mark.parametrize("dtype,ydtype", [(torch.bfloat16, torch.bfloat16), (torch.float32, torch.float32),
                                          (torch.float32, torch.bfloat16), (torch.bfloat16, torch.float32)])
def test_add_rmsnorm_equals_two_calls(lib, dtype, ydtype):
    # bi_add_rmsnorm == bi_residual_add then bi_rmsnorm, both outputs bit for bit, including
    # the sum written over one of its inputs
    rng = np.random.default_rng(11)
    for m, d in [(1, 4096), (7, 512), (300, 4096), (3, 8192), (5, 1032)]:
        say("add + rmsnorm", m, d, dtype, ydtype)
        a = torch.from_numpy(rng.standard_normal((m, d)).astype(np.float32)).cuda().to(dtype)
        b = torch.from_numpy((rng.standard_normal((m, d)) * 0.3).astype(np.float32)).cuda().to(dtype)
        g = bf16(normal_bf16((d,), 1.0, 0.02, 12, d))
        s_ref = lib.bi_residual_add(a, b)
        y_ref = lib.bi_rmsnorm(s_ref, g, 1e-5, out_dtype=ydtype)
        s_got, y_got = lib.bi_add_rmsnorm(a, b, g, 1e-5, out_dtype=ydtype)
        assert same_bits(s_got, s_ref) and same_bits(y_got, y_ref), (m, d)
        a2 = a.clone()
        s2, y2 = lib.bi_add_rmsnorm(a2, b, g, 1e-5, sum_out=a2, out_dtype=ydtype)
        assert same_bits(s2, s_ref) and same_bits(y2, y_ref), (m, d)


@pytest.mark.parametrize("m,d", [(9001, 4096), (9001, 8192), (20011, 512), (17003, 104)])
def test_many_rows_bit_exact(lib, m, d):
    # thousands of rows (many more workgroups than can be resident, row counts that are not
    # a multiple of anything): every row equals the oracle's tree replay, and the same row
    # computed alone
    say("rmsnorm many rows", m, d)
    x = normal_bf16((m, d), 0.0, 1.0, 25, d)
    g = normal_bf16((d,), 1.0, 0.02, 25, d + 1)
    X, G = bf16(x), bf16(g)
    y = lib.bi_rmsnorm(X, G, 1e-5)
    assert np.array_equal(bits(y), rmsnorm_tree(x, g, 1e-5))
    for r in (0, 1, m // 2, m - 1):
        assert same_bits(lib.bi_rmsnorm(X[r:r + 1], G, 1e-5)[0], y[r])
