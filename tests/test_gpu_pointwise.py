"""The pointwise glue on the GPU against the oracle, each op on its own inputs: RoPE with the
q/k/v split, SwiGLU, the residual add, the embedding gather, the fused gate/up + SwiGLU GEMM
and the fused residual add + RMSNorm.

Cited: "Defeating nondeterminism in LLM inference", section on making kernels
batch-invariant (pointwise operations run the same code per element); readings for RoPE
(rotate-half pairing, base 10000, fp64 angles) and SwiGLU in oracle/layer.py.
Bars: within 1 bf16 ulp at output scale of the fp64 formula rounded once (RoPE, SwiGLU),
bit-exact where the result is one rounding of an exact value (residual add, gather, RMSNorm
tree replay); the fused GEMM inside the interval its projection's 1-ulp bar allows.
"""
import numpy as np
import pytest
import torch

from oracle import fp
from oracle.check import bf16_within_1ulp, f32_within_rel, swiglu_interval_within
from oracle.gemm import gemm_f64
from oracle.layer import Spec, op_rope_qkv, store, swiglu_f64
from oracle.rmsnorm import rmsnorm_tree
from synth import gemm_inputs, normal_bf16, uniform_ints
from tests._gpu import bf16, bits, f32, host, i32, same_bits, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("T,hq,hkv,hd,qkv_f32", [(7, 32, 8, 128, False), (300, 32, 8, 128, False),
                                                (5, 32, 8, 128, True), (260, 4, 2, 64, True),
                                                (1, 8, 8, 16, False)])
def test_rope_qkv_vs_oracle(lib, T, hq, hkv, hd, qkv_f32):
    # positions across the 32k context (0, chunk and group boundaries, the last positions)
    # plus random ones; under and over 256 tokens (one head per thread, or eight)
    say("rope", T, hq, hkv, hd, "fp32 qkv" if qkv_f32 else "bf16 qkv")
    width = (hq + 2 * hkv) * hd
    fixed = [0, 1, 255, 256, 1023, 1024, 16383, 16384, 32766, 32767]
    pos = np.concatenate([fixed, uniform_ints(T, 0, 32767, 60, T)])[:T].astype(np.int32)
    if qkv_f32:
        x = np.random.default_rng(T).standard_normal((T, width)).astype(np.float32) * 2
        qkv = f32(x)
        x64 = x.astype(np.float64)
    else:
        xb = normal_bf16((T, width), 0, 2.0, 60, 1000 + T)
        qkv = bf16(xb)
        x64 = fp.bf16_to_f64(xb)
    q, k, v = lib.bi_rope_qkv(qkv, i32(pos), hq, hkv, hd, 10000.0)
    spec = Spec(n_q_heads=hq, n_kv_heads=hkv, head_dim=hd)
    q64, k64, v64 = op_rope_qkv(x64, pos, spec)
    # q kept in fp32 (the FP32-activation variant): within 1e-3 at output scale, and its
    # bf16 rounding is the bf16 call's q
    q32, k2, _ = lib.bi_rope_qkv(qkv, i32(pos), hq, hkv, hd, 10000.0, q_dtype=torch.float32)
    r32 = f32_within_rel(host(q32), q64)
    assert r32["ok"] and r32["max_rel"] < 1e-5, r32
    assert same_bits(q32.to(torch.bfloat16), q) and same_bits(k2, k)
    rq = bf16_within_1ulp(bits(q), q64)
    rk = bf16_within_1ulp(bits(k), k64)
    say("rope q", rq, "k", rk)
    assert rq["ok"] and rk["ok"], (rq, rk)
    assert np.array_equal(bits(v), fp.f64_to_bf16(v64))
    # position 0 is the identity rotation (exactly the rounded input)
    if pos[0] == 0:
        assert np.array_equal(bits(q)[0], fp.f64_to_bf16(x64[0, :hq * hd].reshape(hq, hd)))


def test_rope_is_per_token(lib):
    # a token's rotation does not depend on the other tokens of the call
    xb = normal_bf16((300, 48 * 128), 0, 1.0, 61, 0)
    pos = uniform_ints(300, 0, 32767, 61, 1).astype(np.int32)
    q, k, _ = lib.bi_rope_qkv(bf16(xb), i32(pos), 32, 8, 128, 10000.0)
    for sel in ([0], [17, 3], list(range(100, 103))):
        q1, k1, _ = lib.bi_rope_qkv(bf16(xb[sel]), i32(pos[sel]), 32, 8, 128, 10000.0)
        assert same_bits(q1, q[sel]) and same_bits(k1, k[sel])


def test_swiglu_vs_oracle(lib):
    gu = normal_bf16((33, 2 * 1000), 0, 2.0, 62, 0)
    gu[0, :8] = fp.f32_to_bf16(np.float32([0.0, -0.0, 1.0, -1.0, 20.0, -20.0, 80.0, -80.0]))
    out = lib.bi_swiglu(bf16(gu))
    g64 = fp.bf16_to_f64(gu)
    ref = swiglu_f64(g64[:, :1000], g64[:, 1000:])
    r = bf16_within_1ulp(bits(out), ref)
    say("swiglu", r)
    assert r["ok"], r
    assert np.array_equal(bits(out)[0, :2], fp.f64_to_bf16(ref[0, :2]))   # silu(0) u = 0


@pytest.mark.parametrize("dt", [("bf16", "bf16", "bf16"), ("f32", "bf16", "f32"), ("bf16", "f32", "bf16"),
                                ("f32", "f32", "f32"), ("bf16", "bf16", "f32")])
def test_residual_add_bit_exact(lib, dt):
    # the contract: an fp32 add (one rounding of the exact sum), then one rounding to the
    # output type -- for two bf16 operands that is one rounding of the exact sum to any type
    n = 4096 * 3 + 8
    rng = np.random.default_rng(63)
    vals = {}
    for name, d in zip("ab", dt[:2]):
        x = (rng.standard_normal(n) * rng.choice([1e-3, 1.0, 300.0], n)).astype(np.float32)
        vals[name] = (bf16(fp.f32_to_bf16(x)), fp.bf16_to_f64(fp.f32_to_bf16(x))) if d == "bf16" else \
            (f32(x), x.astype(np.float64))
    out_dtype = torch.bfloat16 if dt[2] == "bf16" else torch.float32
    for length in (n, n - 3):      # the 8-wide bf16 kernel and the element kernel
        a, b = vals["a"][0][:length], vals["b"][0][:length]
        got = lib.bi_residual_add(a, b, out_dtype=out_dtype)
        want = store(store(vals["a"][1][:length] + vals["b"][1][:length], "f32"), dt[2])
        if dt[:2] == ("bf16", "bf16"):
            assert np.array_equal(want, store(vals["a"][1][:length] + vals["b"][1][:length], dt[2]))
        g = fp.bf16_to_f64(bits(got)) if dt[2] == "bf16" else host(got).astype(np.float64)
        assert np.array_equal(g, want), (dt, length)


def test_embedding_gather(lib):
    table = normal_bf16((1000, 256), 0, 0.02, 64, 0)
    ids = np.asarray([0, 999, 5, 5, 1000, -1, 17], dtype=np.int32)
    out = lib.bi_embedding(i32(ids), bf16(table))
    want = np.zeros((7, 256), dtype=np.uint16)
    ok = (ids >= 0) & (ids < 1000)
    want[ok] = table[ids[ok]]
    assert np.array_equal(bits(out), want)
    wide = lib.bi_embedding(i32(ids), bf16(table), out_dtype=torch.float32)
    assert np.array_equal(host(wide), fp.bf16_to_f32(want))
    # an fp32 table gathered into bf16: one rounding per element
    tf = np.random.default_rng(64).standard_normal((50, 64)).astype(np.float32)
    got = lib.bi_embedding(i32([3, 49]), f32(tf))
    assert np.array_equal(bits(got), fp.f32_to_bf16(tf[[3, 49]]))


@pytest.mark.parametrize("f,k", [(14336, 4096), (1024, 1024), (3008, 1000)])
def test_gemm_swiglu_vs_oracle(lib, f, k):
    # the fused gate/up projection + SwiGLU against the oracle's fp64 projection, at row
    # counts that select the few-row waves (paired and two-block), the mid tiles and the
    # 128 x 128 / 256 x 256 tiles
    from invariant_amd import interleave_gate_up
    a, b = gemm_inputs(1100, 2 * f, k, cfg=65, sd=0.5)
    W = bf16(np.ascontiguousarray(b.T))
    Wi = interleave_gate_up(W)
    A = bf16(a)
    for m in (1, 8, 9, 40, 300, 1100):
        say("gemm_swiglu", f, k, m, lib.bi_gemm_tile(m, 2 * f, k))
        out = lib.bi_gemm_swiglu(A[:m], Wi)
        ref = gemm_f64(a[:m], b)
        r = swiglu_interval_within(bits(out), ref[:, :f], ref[:, f:])
        assert r["ok"], (m, r)


def test_add_rmsnorm_vs_oracle(lib):
    # the fused residual add + RMSNorm: the sum is one rounding of the exact sum, the norm the
    # tree replay of that rounded sum (bf16 and fp32 residual streams)
    a = normal_bf16((70, 4096), 0, 1.0, 66, 0)
    b = normal_bf16((70, 4096), 0, 0.3, 66, 1)
    g = normal_bf16((4096,), 1.0, 0.02, 66, 2)
    s, y = lib.bi_add_rmsnorm(bf16(a), bf16(b), bf16(g), 1e-5)
    s_ref = fp.f64_to_bf16(fp.bf16_to_f64(a) + fp.bf16_to_f64(b))
    assert np.array_equal(bits(s), s_ref)
    assert np.array_equal(bits(y), rmsnorm_tree(s_ref, g, 1e-5))
    af = fp.bf16_to_f32(a) * np.float32(1.0 + 2 ** -12)
    s, y = lib.bi_add_rmsnorm(f32(af), f32(fp.bf16_to_f32(b)), bf16(g), 1e-5, out_dtype=torch.float32)
    s_ref = (af.astype(np.float64) + fp.bf16_to_f64(b)).astype(np.float32)
    assert np.array_equal(host(s), s_ref)
    assert np.array_equal(host(y), rmsnorm_tree(s_ref, g, 1e-5, "f32", "f32"))
