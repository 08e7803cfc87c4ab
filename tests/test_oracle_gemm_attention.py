"""Pins of the GEMM and attention oracles (CPU only).

Cited: "Defeating nondeterminism in LLM inference": introduction (torch.mm), sections
"batch-invariant matrix multiplication" and "batch-invariant attention" (reduction
over feature and sequence dimensions; KV cache written before attention).
"""
import numpy as np

from oracle import fp
from oracle.attention import attention_rows_f64, attention_case_f64
from oracle.gemm import gemm_f64
from synth import attention_case, normal_bf16
from tests import _scalar_ref as S


def test_gemm_brute_force_fraction_both_layouts():
    for m, k, n, seed in [(3, 5, 7, 0), (17, 33, 9, 1), (1, 64, 2, 2)]:
        a = normal_bf16((m, k), 0, 1, 900, seed)
        b = normal_bf16((k, n), 0, 1, 901, seed)
        exact = S.matmul_fraction(fp.bf16_to_f64(a).tolist(), fp.bf16_to_f64(b).tolist())
        exact = np.array([[float(v) for v in row] for row in exact])
        got_kn = gemm_f64(a, b, "kn")
        got_nk = gemm_f64(a, np.ascontiguousarray(b.T), "nk")
        assert np.max(np.abs(got_kn - exact)) <= 1e-12 * np.abs(exact).max()
        assert np.array_equal(got_kn, got_nk)


def test_gemm_fp32_operand_exact():
    a = np.float32([[1.0 + 2 ** -20, 3.0], [-2.0, 0.5]])
    b = fp.f32_to_bf16(np.float32([[1.0, 2.0], [4.0, -1.0]]))
    got = gemm_f64(a, b, "kn", a_dtype="f32")
    assert got[0, 0] == 1.0 + 2 ** -20 + 12.0 and got[1, 1] == -4.5


def test_attention_matches_scalar_brute_force():
    case = attention_case([5, 9], [5, 2], n_q_heads=4, n_kv_heads=2, head_dim=8, cfg=910)
    outs = attention_case_f64(case)
    for b, (L, ql) in enumerate(zip(case["seq_lens"], case["q_lens"])):
        q = fp.bf16_to_f64(case["q"][b]).tolist()
        k = fp.bf16_to_f64(case["k"][b]).tolist()
        v = fp.bf16_to_f64(case["v"][b]).tolist()
        for i in range(ql):
            p = L - ql + i
            ref = np.array(S.attention_scalar(q[i], k, v, p, 2))
            assert np.max(np.abs(outs[b][i] - ref)) < 1e-12


def test_attention_closed_forms():
    L, hq, hkv, d = 40, 8, 2, 16
    rng = np.random.default_rng(0)
    kb = fp.f32_to_bf16(rng.standard_normal((L, hkv, d)).astype(np.float32))
    vb = fp.f32_to_bf16(rng.standard_normal((L, hkv, d)).astype(np.float32))
    # L = 1: the output is v_0 exactly
    q1 = fp.f32_to_bf16(rng.standard_normal((1, hq, d)).astype(np.float32))
    o = attention_rows_f64(q1, kb, vb, [0])
    for h in range(hq):
        assert np.array_equal(o[0, h], fp.bf16_to_f64(vb[0, h // 4]))
    # q = 0: uniform weights, output is the mean of v_0..v_p
    q0 = np.zeros((3, hq, d), dtype=np.uint16)
    o = attention_rows_f64(q0, kb, vb, [3, 17, 39])
    V = fp.bf16_to_f64(vb)
    for i, p in enumerate([3, 17, 39]):
        assert np.allclose(o[i, 5], V[: p + 1, 1].mean(axis=0), rtol=0, atol=1e-14)
    # GQA mapping h -> h // (Hq/Hkv): kv head g carries the constant g + 1
    vg = np.zeros((L, hkv, d), dtype=np.float32)
    for g in range(hkv):
        vg[:, g, :] = g + 1
    o = attention_rows_f64(q1, kb, fp.f32_to_bf16(vg), [20])
    for h in range(hq):
        assert np.allclose(o[0, h], h // 4 + 1, rtol=1e-14, atol=0)
    # identical keys: uniform weights whatever q is
    ksame = np.repeat(kb[:1], L, axis=0)
    o = attention_rows_f64(q1, ksame, vb, [9])
    assert np.allclose(o[0, 0], V[:10, 0].mean(axis=0), atol=1e-14)


def test_attention_is_causal():
    case = attention_case([600], [600], n_q_heads=4, n_kv_heads=1, head_dim=16, cfg=911)
    base = attention_case_f64(case, which={0: [100, 300]})[0]
    case["k"][0][301:] = 0x3F80
    case["v"][0][301:] = 0x4000
    after = attention_case_f64(case, which={0: [100, 300]})[0]
    assert np.array_equal(base, after)
