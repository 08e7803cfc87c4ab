"""bi_gemm on the GPU: within 1 bf16 ulp (at output scale) of the fp64 oracle, bit-exact
when every order is exact, and bitwise batch- and position-invariant.

Cited: "Defeating nondeterminism in LLM inference": introduction (repeated torch.mm is
bitwise equal), sections on batch invariance (the linspace example: row 0 of a
[1, D] product vs of a [2048, D] product) and batch-invariant matrix multiplication.
"""
import numpy as np
import pytest
import torch

from oracle import fp
from oracle.check import bf16_within_1ulp, f32_within_rel
from oracle.gemm import gemm_f64
from oracle.rmsnorm import rmsnorm_tree
from synth import gemm_inputs, normal_bf16, rmsnorm_linear_inputs
from tests._gpu import bf16, bits, f32, host, same_bits, say

pytestmark = pytest.mark.gpu


def _nk(b_kn):
    return np.ascontiguousarray(b_kn.T)


def test_identity_b_gives_a(lib):
    a = normal_bf16((70, 96), 0, 1, 30, 0)
    eye = fp.f32_to_bf16(np.eye(96, dtype=np.float32))
    c = lib.bi_gemm(bf16(a), bf16(eye))
    assert np.array_equal(bits(c), a)


@pytest.mark.parametrize("m,n,k", [(1, 512, 512), (33, 200, 72), (128, 128, 64), (130, 260, 1000),
                                   (257, 384, 4096), (512, 1024, 14336), (7, 6144, 4096)])
def test_vs_oracle(lib, m, n, k):
    say("gemm", m, n, k)
    a, b = gemm_inputs(m, n, k, cfg=31)
    c = lib.bi_gemm(bf16(a), bf16(_nk(b)))
    r = bf16_within_1ulp(bits(c), gemm_f64(a, b))
    assert r["ok"], r
    cf = lib.bi_gemm(bf16(a), bf16(_nk(b)), out_dtype=torch.float32)
    r = f32_within_rel(host(cf), gemm_f64(a, b))
    assert r["ok"], r


@pytest.mark.parametrize("m,n,k", [(4096, 4096, 256), (3100, 8000, 200)])
def test_large_tile_vs_oracle(lib, m, n, k):
    # output grids large enough for the 256 x 256 workgroup tile, ragged in M, N and K
    assert lib.bi_gemm_tile(m, n, k)[:2] == (256, 256)
    say("gemm large tile", m, n, k)
    a, b = gemm_inputs(m, n, k, cfg=36)
    c = lib.bi_gemm(bf16(a), bf16(_nk(b)))
    r = bf16_within_1ulp(bits(c), gemm_f64(a, b))
    assert r["ok"], r


def few_rows(m, n, k):
    """Whether the few-row kernel takes an M x N x K product: up to 32 rows, or up to 64 while
    N / 32 <= CUs, with K a multiple of 8 and at least 2 PF whole 32-wide steps (PF = 16 up
    to 16 rows, 12 above)."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    if m > 64 or (m > 32 and (n + 31) // 32 > cus):
        return False
    return k % 8 == 0 and k // 32 >= 2 * (16 if m <= 16 else 12)


def test_tile_switch_changes_no_bit(lib):
    # the same rows computed under every workgroup configuration (256 x 256; 128 x 128 with
    # a 2- or 3-stage ring), chosen by the grid size, at several positions, for a square
    # and a ragged N
    for n, k, full_m in [(4096, 4096, 4096), (6000, 1000, 8192)]:
        a, b = gemm_inputs(full_m, n, k, cfg=37)
        A, B = bf16(a), bf16(_nk(b))
        assert lib.bi_gemm_tile(full_m, n, k)[:2] == (256, 256)
        full = lib.bi_gemm(A, B)
        configs = {lib.bi_gemm_tile(full_m, n, k)}
        for m in (1, 33, 64, 65, 255, 500, 640, 1000, 2048, 2560, 3000):
            configs.add(lib.bi_gemm_tile(m, n, k))
            assert same_bits(lib.bi_gemm(A[:m], B), full[:m]), (n, k, m)
        assert {(64, 64, 3), (64, 128, 3), (128, 128, 3), (128, 128, 2), (256, 256, 2)} <= configs, configs
        # the few-row kernel (16 or 32 columns per wave) where its K condition holds
        for m in (1, 33, 64):
            assert (lib.bi_gemm_tile(m, n, k)[1] <= 32) == few_rows(m, n, k), (m, n, k)
        sel = torch.tensor([full_m - 1, 17, 2600, 300], device="cuda")
        assert same_bits(lib.bi_gemm(A[sel].contiguous(), B), full[sel])
        ff = lib.bi_gemm(A, B, out_dtype=torch.float32)
        assert same_bits(lib.bi_gemm(A[sel].contiguous(), B, out_dtype=torch.float32), ff[sel])


def test_integer_inputs_bit_exact(lib):
    rng = np.random.default_rng(0)
    a = fp.f32_to_bf16(rng.integers(-8, 9, (300, 1000)).astype(np.float32))
    b = fp.f32_to_bf16(rng.integers(-8, 9, (1000, 200)).astype(np.float32))
    ref = gemm_f64(a, b)
    assert np.abs(ref).max() < 2 ** 24
    c = lib.bi_gemm(bf16(a), bf16(_nk(b)), out_dtype=torch.float32)
    assert np.array_equal(host(c).astype(np.float64), ref)


def test_rmsnorm_then_512_linear_batch_sweep(lib):
    x, gamma, w = rmsnorm_linear_inputs(32, 512, 512)
    X, G, W = bf16(x), bf16(gamma), bf16(w)
    row0 = None
    for m in range(1, 33):
        y = lib.bi_rmsnorm(X[:m], G, 1e-6)
        z = lib.bi_gemm(y, W)
        yr = rmsnorm_tree(x[:m], gamma, 1e-6)
        ref = gemm_f64(yr, w, "nk")
        r = bf16_within_1ulp(bits(z), ref)
        assert r["ok"], (m, r)
        row0 = z[0].clone() if row0 is None else row0
        assert same_bits(z[0], row0), m


def test_gemm_2048_repeats_prefixes_permutation(lib):
    a, b = gemm_inputs(2048, 2048, 2048, cfg=2)
    A, B = bf16(a), bf16(_nk(b))
    ref = lib.bi_gemm(A, B)
    torch.cuda.synchronize()
    r = bf16_within_1ulp(bits(ref[:64]), gemm_f64(a[:64], b))
    assert r["ok"], r
    for _ in range(1000):
        c = lib.bi_gemm(A, B)
        assert (c.float() - ref.float()).abs().max().item() == 0
    for m in (1, 3, 17, 128, 511, 2048):
        assert same_bits(lib.bi_gemm(A[:m], B), ref[:m]), m
    perm = torch.randperm(2048, generator=torch.Generator().manual_seed(0)).cuda()
    assert same_bits(lib.bi_gemm(A[perm].contiguous(), B), ref[perm])
    # rows placed mid-batch among other rows
    mix = torch.cat([A[100:101], torch.randn(40, 2048, device="cuda").to(torch.bfloat16), A[5:6]])
    cm = lib.bi_gemm(mix, B)
    assert same_bits(cm[0], ref[100]) and same_bits(cm[41], ref[5])


def test_gemm_2048_torch_mm_orientation(lib):
    # the 2048^3 product in the orientation of the page's torch.mm(A, B): B is [K, N] as drawn.  1000
    # repeats are bitwise equal, prefix rows equal the full product's rows, and every bit
    # equals the [N, K] layout's result on the transposed copy of B (same instruction
    # sequence per element)
    from invariant_amd import BI_B_KN
    a, b = gemm_inputs(2048, 2048, 2048, cfg=2)
    A, Bkn = bf16(a), bf16(b)
    ref = lib.bi_gemm(A, Bkn, b_layout=BI_B_KN)
    assert same_bits(ref, lib.bi_gemm(A, bf16(_nk(b))))
    r = bf16_within_1ulp(bits(ref[:64]), gemm_f64(a[:64], b))
    assert r["ok"], r
    for _ in range(1000):
        c = lib.bi_gemm(A, Bkn, b_layout=BI_B_KN)
        assert (c.float() - ref.float()).abs().max().item() == 0
    for m in (1, 3, 17, 128, 511, 2048):
        assert same_bits(lib.bi_gemm(A[:m], Bkn, b_layout=BI_B_KN), ref[:m]), m
    perm = torch.randperm(2048, generator=torch.Generator().manual_seed(1)).cuda()
    assert same_bits(lib.bi_gemm(A[perm].contiguous(), Bkn, b_layout=BI_B_KN), ref[perm])


@pytest.mark.parametrize("m,n,k", [(1, 1003, 77), (33, 200, 1000), (300, 8, 4096), (130, 4100, 64),
                                   (3000, 700, 300), (1, 512, 4096), (600, 4096, 1000),
                                   (4096, 4096, 256), (2048, 2048, 2048)])
def test_b_kn_ragged_equals_b_nk(lib, m, n, k):
    # [K, N] B with N off a multiple of 8 (row stride padded to one, the padding NaN: nothing
    # past column N may be read into a stored output) and ragged K: bits of the [N, K] layout,
    # within 1 ulp of the oracle, for bf16 and fp32 A; with bf16 A the shapes reach every
    # tile the [K, N] form takes (64 x 64, 64 x 128, 128 x 128 one and two per CU)
    from invariant_amd import BI_B_KN
    say("gemm B [K, N]", m, n, k)
    a, b = gemm_inputs(m, n, k, cfg=46)
    ldb = (n + 7) // 8 * 8 + 8
    Bp = torch.full((k, ldb), float("nan"), device="cuda").to(torch.bfloat16)
    Bp[:, :n] = bf16(b)
    Bkn = Bp[:, :n]
    def padded(x):     # row stride a multiple of 8 elements, as bi_gemm requires
        r, c_ = x.shape
        p = torch.zeros((r, (c_ + 7) // 8 * 8 + 8), dtype=torch.bfloat16, device="cuda")
        p[:, :c_] = bf16(x)
        return p[:, :c_]
    A = padded(a)
    Bnk = padded(_nk(b))
    c = lib.bi_gemm(A, Bkn, b_layout=BI_B_KN)
    assert same_bits(c, lib.bi_gemm(A, Bnk))
    r = bf16_within_1ulp(bits(c), gemm_f64(a, b))
    assert r["ok"], r
    cf = lib.bi_gemm(A, Bkn, b_layout=BI_B_KN, out_dtype=torch.float32)
    assert same_bits(cf, lib.bi_gemm(A, Bnk, out_dtype=torch.float32))
    afp = torch.zeros((m, (k + 3) // 4 * 4 + 4), device="cuda")
    afp[:, :k] = bf16(a).float()
    af = afp[:, :k]
    c32 = lib.bi_gemm(af, Bkn, b_layout=BI_B_KN, out_dtype=torch.float32)
    assert same_bits(c32, lib.bi_gemm(af, Bnk, out_dtype=torch.float32))


def _padded(x):
    """bf16 copy of x whose rows have a stride of a multiple of 8 elements with zero padding
    (every row readable in whole 16-byte pieces, the last one included)."""
    r, c_ = x.shape
    p = torch.zeros((r, (c_ + 7) // 8 * 8), dtype=torch.bfloat16, device="cuda")
    p[:, :c_] = bf16(x)
    return p[:, :c_]


@pytest.mark.parametrize("m,n,k", [(1, 1, 1), (1, 17, 1), (300, 3, 1), (3, 5, 7), (17, 1, 33),
                                   (2, 3, 31), (64, 2, 8), (1, 1, 4100)])
def test_degenerate_shapes(lib, m, n, k):
    # one output row or column, K under one 8-element piece or one 32-wide step.  At K = 1
    # every output is one product of two bf16 values (exact in fp32) rounded once, so bf16
    # and fp32 outputs equal the fp64 oracle rounded once, bit for bit; otherwise the 1-ulp
    # bar.  The [K, N] layout gives the [N, K] bits.
    from invariant_amd import BI_B_KN
    say("gemm degenerate", m, n, k)
    a, b = gemm_inputs(m, n, k, cfg=38)
    A, Bnk, Bkn = _padded(a), _padded(_nk(b)), _padded(b)
    ref = gemm_f64(a, b)
    c = lib.bi_gemm(A, Bnk)
    cf = lib.bi_gemm(A, Bnk, out_dtype=torch.float32)
    if k == 1:
        assert np.array_equal(bits(c), fp.f64_to_bf16(ref))
        assert np.array_equal(host(cf), ref.astype(np.float32))
    else:
        r = bf16_within_1ulp(bits(c), ref)
        assert r["ok"], r
        assert f32_within_rel(host(cf), ref)["ok"]
    assert same_bits(lib.bi_gemm(A, Bkn, b_layout=BI_B_KN), c)
    # each row alone: the same bits
    for i in sorted({0, m - 1}):
        assert same_bits(lib.bi_gemm(A[i:i + 1], Bnk), c[i:i + 1])


def test_splitk_variant_is_not_invariant(lib):
    # the page's linspace example: row 0 of a [1, D] product vs of a [2048, D] product
    Bn, D = 2048, 4096
    a = torch.linspace(-1000, 1000, Bn * D, device="cuda").reshape(Bn, D).to(torch.bfloat16)
    b = torch.linspace(-1000, 1000, D * D, device="cuda").reshape(D, D).to(torch.bfloat16)
    bt = b.t().contiguous()
    inv1 = lib.bi_gemm(a[:1], bt, out_dtype=torch.float32)
    inv2 = lib.bi_gemm(a, bt, out_dtype=torch.float32)[:1]
    assert (inv1 - inv2).abs().max().item() == 0
    s1 = lib.bi_gemm_splitk(a[:1], bt, out_dtype=torch.float32)
    s2 = lib.bi_gemm_splitk(a, bt, out_dtype=torch.float32)[:1]
    say("split-K row-0 max diff", (s1 - s2).abs().max().item())
    assert (s1 - s2).abs().max().item() > 0
    # on well-conditioned data the split-K variant is still a correct GEMM
    a2, b2 = gemm_inputs(64, 512, 4096, cfg=34)
    sk = lib.bi_gemm_splitk(bf16(a2), bf16(_nk(b2)))
    assert bf16_within_1ulp(bits(sk), gemm_f64(a2, b2))["ok"]


def test_splitk_variant_vs_oracle_and_slices(lib):
    # the comparison variant on the few-row and the LDS-staged kernels, with slice counts
    # that change with M: a correct GEMM on well-conditioned data, not an invariant one
    a, b = gemm_inputs(1000, 1024, 4096, cfg=48, sd=1.0)
    A, W = bf16(a), bf16(np.ascontiguousarray(b.T))
    slices = set()
    for m in (1, 33, 64, 300, 1000):
        need = lib.load().bi_gemm_splitk_workspace_bytes(m, 1024, 4096)
        slices.add(max(1, need // (4 * m * 1024)))
        c = lib.bi_gemm_splitk(A[:m], W)
        r = bf16_within_1ulp(bits(c), gemm_f64(a[:m], b))
        assert r["ok"], (m, r)
    say("split-K slice counts over M", sorted(slices))
    assert len(slices) > 1
    # up to 4 rows: K split over the 4 waves of a workgroup (segments of 8, 16, 32 steps,
    # whole steps past K skipped, a partial last step, ragged N)
    for n, k in ((1024, 1000), (300, 520), (4100, 3000), (6144, 4096)):
        a, b = gemm_inputs(4, n, k, cfg=50)
        W = bf16(np.ascontiguousarray(b.T))
        for m in (1, 2, 4):
            c = lib.bi_gemm_splitk(bf16(a[:m]), W)
            r = bf16_within_1ulp(bits(c), gemm_f64(a[:m], b))
            assert r["ok"], (n, k, m, r)


def test_fp32_operand_variant(lib):
    rng = np.random.default_rng(2)
    af = rng.standard_normal((100, 4096)).astype(np.float32)
    w = normal_bf16((300, 4096), 0, 0.02, 32, 0)
    c = lib.bi_gemm(f32(af), bf16(w), out_dtype=torch.float32)
    ref = gemm_f64(af, w, "nk", a_dtype="f32")
    r = f32_within_rel(host(c), ref)
    assert r["ok"], r
    # the fp32-operand path is far closer than rounding the operand to bf16 first
    ab = lib.bi_gemm(f32(af).to(torch.bfloat16), bf16(w), out_dtype=torch.float32)
    err32 = np.abs(host(c) - ref).max()
    err16 = np.abs(host(ab) - ref).max()
    say("fp32-operand max err", err32, "bf16-operand max err", err16)
    assert err32 * 8 < err16
    # exact split: a value with all 24 mantissa bits times 1.0 comes back exactly
    a1 = np.float32([[1.0 + 2 ** -23 + 2 ** -10, -3.1415927]] + [[0.0, 0.0]] * 7)
    e = fp.f32_to_bf16(np.eye(2, 8, dtype=np.float32)[:2, :2])
    a8 = np.zeros((8, 8), dtype=np.float32); a8[:, :2] = a1
    w8 = np.zeros((2, 8), dtype=np.uint16); w8[:, :2] = e
    c1 = lib.bi_gemm(f32(a8), bf16(w8), out_dtype=torch.float32)
    assert np.array_equal(host(c1)[0], a1[0])
    # batch invariance of the fp32 path
    A = f32(af)
    full = lib.bi_gemm(A, bf16(w), out_dtype=torch.float32)
    assert same_bits(lib.bi_gemm(A[:1], bf16(w), out_dtype=torch.float32)[0], full[0])


def test_k_tail_with_garbage_past_k(lib):
    # rows padded to a multiple of 8 elements, the padding filled with NaN: every product
    # past K must be an exact zero
    for m, n, k in [(65, 70, 1003), (3, 130, 77), (200, 33, 9), (3100, 8000, 77), (1000, 600, 50)]:
        a, b = gemm_inputs(m, n, k, cfg=35)
        kp = (k + 7) // 8 * 8 + 8
        A = torch.full((m, kp), float("nan"), device="cuda").to(torch.bfloat16)
        W = torch.full((n, kp), float("nan"), device="cuda").to(torch.bfloat16)
        A[:, :k] = bf16(a)
        W[:, :k] = bf16(_nk(b))
        c = lib.bi_gemm(A[:, :k], W[:, :k])
        r = bf16_within_1ulp(bits(c), gemm_f64(a, b))
        assert r["ok"], (m, n, k, r)


def test_empty_and_ragged(lib):
    A = torch.zeros((0, 64), dtype=torch.bfloat16, device="cuda")
    W = torch.zeros((16, 64), dtype=torch.bfloat16, device="cuda")
    assert lib.bi_gemm(A, W).shape == (0, 16)
    a, b = gemm_inputs(1, 1, 8, cfg=33)
    c = lib.bi_gemm(bf16(a), bf16(_nk(b)), out_dtype=torch.float32)
    assert f32_within_rel(host(c), gemm_f64(a, b))["ok"]


def test_output_views(lib):
    # C written into row-strided views: 16-byte-aligned rows with a ragged last chunk, and rows
    # that start off 16-byte alignment; every element equals the contiguous result and nothing
    # outside the view changes (grids for the 128 x 128 and the 256 x 256 tiles)
    sentinel = -7.0
    for m, n, k in [(300, 1003, 64), (1000, 600, 56), (3100, 8000, 80), (4096, 4092, 40)]:
        say("gemm output views", m, n, k)
        a, b = gemm_inputs(m, n, k, cfg=38)
        A, W = bf16(a), bf16(_nk(b))
        ref = lib.bi_gemm(A, W)
        for lo, width in [(0, (n + 7) // 8 * 8 + 8), (1, n + 5)]:
            big = torch.full((m, width), sentinel, dtype=torch.bfloat16, device="cuda")
            out = big[:, lo:lo + n]
            lib.bi_gemm(A, W, out=out)
            assert same_bits(out.contiguous(), ref), (m, n, k, lo)
            rest = torch.ones_like(big, dtype=torch.bool)
            rest[:, lo:lo + n] = False
            assert bool((big[rest] == sentinel).all()), (m, n, k, lo)


@pytest.mark.parametrize("m,n,k", [(5, 300, 1024), (40, 1000, 784), (64, 96, 1024), (1, 33, 1040),
                                   (17, 200, 1064), (33, 1000, 1024), (50, 72, 800), (9, 5000, 1024),
                                   (49, 6200, 808), (24, 4096, 1048), (33, 2048, 1032)])
def test_few_rows_vs_oracle(lib, m, n, k):
    # the few-row kernel (M <= 64: 16 x 16, 16 x 32, 32 x 32 or 64 x 32 blocks, two or four
    # waves of 16- or 32-row slices per column block for narrow N, up to one per CU): ragged column blocks, rows past M, padded
    # grids, the last partial round of prefetched K steps, a partial last K step (K % 32 = 8,
    # 16)
    assert lib.bi_gemm_tile(m, n, k)[1] <= 32
    say("gemm few rows", m, n, k)
    a, b = gemm_inputs(m, n, k, cfg=39)
    c = lib.bi_gemm(bf16(a), bf16(_nk(b)))
    r = bf16_within_1ulp(bits(c), gemm_f64(a, b))
    assert r["ok"], r
    cf = lib.bi_gemm(bf16(a), bf16(_nk(b)), out_dtype=torch.float32)
    r = f32_within_rel(host(cf), gemm_f64(a, b))
    assert r["ok"], r


@pytest.mark.parametrize("n,k", [(4096, 4096), (28672, 1024), (6144, 14336), (32000, 512), (2048, 1024),
                                 (1024, 4096)])
def test_few_rows_match_large_m(lib, n, k):
    # the few-row kernel (every block shape and row split) gives the rows of the large-M
    # kernels bit for bit
    say("gemm few rows vs large M", n, k)
    a, b = gemm_inputs(512, n, k, cfg=40)
    A, W = bf16(a), bf16(_nk(b))
    full = lib.bi_gemm(A, W)
    ff = lib.bi_gemm(A, W, out_dtype=torch.float32)
    for m in (1, 16, 17, 32, 33, 49, 64):
        assert (lib.bi_gemm_tile(m, n, k)[1] <= 32) == few_rows(m, n, k), (m, n, k)
        assert same_bits(lib.bi_gemm(A[:m], W), full[:m]), (n, k, m)
        assert same_bits(lib.bi_gemm(A[:m], W, out_dtype=torch.float32), ff[:m]), (n, k, m)
    rows = torch.tensor([300, 5, 511], device="cuda")
    assert same_bits(lib.bi_gemm(A[rows].contiguous(), W), full[rows])


@pytest.mark.parametrize("f,k", [(14336, 4096), (3008, 1000), (48, 512), (1024, 1024)])
def test_gemm_swiglu_equals_unfused(lib, f, k):
    # bi_gemm_swiglu with the 16-row interleaved weight == bi_swiglu(bi_gemm(., gate-then-up
    # weight)) bit for bit, for row counts that select every GEMM configuration
    from invariant_amd import interleave_gate_up
    say("gemm + swiglu fused", f, k)
    a, b = gemm_inputs(3000, 2 * f, k, cfg=45, sd=0.5)
    A, W = bf16(a), bf16(_nk(b))
    Wi = interleave_gate_up(W)
    for m in (1, 8, 9, 17, 33, 64, 65, 255, 500, 1000, 3000):
        fused = lib.bi_gemm_swiglu(A[:m], Wi)
        ref = lib.bi_swiglu(lib.bi_gemm(A[:m], W))
        assert same_bits(fused, ref), (f, k, m, lib.bi_gemm_tile(m, 2 * f, k))
    # row-strided, unaligned output view; nothing outside it changes
    big = torch.full((300, f + 5), -3.0, dtype=torch.bfloat16, device="cuda")
    lib.bi_gemm_swiglu(A[:300], Wi, out=big[:, 1:f + 1])
    assert same_bits(big[:, 1:f + 1].contiguous(), lib.bi_swiglu(lib.bi_gemm(A[:300], W)))
    assert bool((big[:, 0] == -3.0).all()) and bool((big[:, f + 1:] == -3.0).all())


def _pack_host(b_nk):
    """The tiled layout of bi_pack_b written out on the host (include/bi.h, BI_B_TILED)."""
    n, k = b_nk.shape
    nb, nt = -(-n // 16), -(-k // 32)
    full = np.zeros((nb * 16, nt * 32), dtype=np.uint16)
    full[:n, :k] = b_nk
    # [b, r, t, g, e] -> [b, t, g, r, e]: lane = r + 16 g
    return full.reshape(nb, 16, nt, 4, 8).transpose(0, 2, 3, 1, 4).reshape(nb, nt, 64, 8)


@pytest.mark.parametrize("n,k", [(4096, 4096), (1000, 1032), (6144, 4096), (32000, 4096),
                                 (4096, 14336), (33, 1024)])
def test_tiled_b_equals_nk(lib, n, k):
    # a tiled B (bi_pack_b) at the row counts the few-row kernel takes it for (up to 64): the
    # bits of the [N, K] call, bf16 and fp32 outputs; ragged N and K (a partial last block and
    # step)
    from invariant_amd import BI_B_TILED
    say("gemm tiled B", n, k)
    a, b = gemm_inputs(64, n, k, cfg=39)
    A, W = bf16(a), bf16(_nk(b))
    Wt = lib.bi_pack_b(W)
    if n * k <= 6144 * 4096:
        assert np.array_equal(bits(Wt), _pack_host(_nk(b)))
    # every few-row configuration: one- and two-block waves, 16-row slices, 32 x 32 and
    # 64 x 32 blocks (above 32 rows on grids wider than the CUs the [N, K] call takes the
    # LDS-staged tiles instead: same bits)
    for m in (1, 3, 8, 9, 16, 17, 24, 32, 33, 49, 64):
        for od in (torch.bfloat16, torch.float32):
            got = lib.bi_gemm(A[:m], Wt, b_layout=BI_B_TILED, n=n, out_dtype=od)
            assert same_bits(got, lib.bi_gemm(A[:m], W, out_dtype=od)), (m, od)
    r = bf16_within_1ulp(bits(lib.bi_gemm(A[:1], Wt, b_layout=BI_B_TILED, n=n)), gemm_f64(a[:1], b))
    assert r["ok"], r


@pytest.mark.parametrize("f,k", [(14336, 4096), (1024, 1024), (3008, 1032)])
def test_tiled_swiglu_equals_interleaved(lib, f, k):
    # the fused gate/up + SwiGLU on the tiled interleaved weights: the bits of the [2F, K] call
    # (paired one-block waves up to 8 rows, two-block waves above, 32 x 32 and 64 x 32 blocks
    # from 17 rows)
    from invariant_amd import BI_B_TILED, interleave_gate_up
    say("gemm_swiglu tiled", f, k)
    a, b = gemm_inputs(64, 2 * f, k, cfg=40, sd=0.5)
    A = bf16(a)
    Wi = interleave_gate_up(bf16(np.ascontiguousarray(b.T)))
    Wt = lib.bi_pack_b(Wi)
    for m in (1, 5, 8, 9, 16, 17, 32, 33, 49, 64):
        got = lib.bi_gemm_swiglu(A[:m], Wt, w_layout=BI_B_TILED)
        assert same_bits(got, lib.bi_gemm_swiglu(A[:m], Wi)), m
