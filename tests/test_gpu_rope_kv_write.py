"""bi_rope_kv_write (RoPE fused with the KV-cache write) on the GPU: the queries, every byte
of both caches and the attention output that follows equal, bit for bit, those of the
unfused calls (bi_rope_qkv, then bi_attention writing k_new / v_new itself), which the
RoPE and attention tests grade against the oracle.

Cited: "Defeating nondeterminism in LLM inference", section on making kernels
batch-invariant (pointwise work fused with its neighbours runs the same code per element)
and section on batch-invariant attention (the cache is written before the kernel reads it).
"""
import numpy as np
import pytest
import torch

from oracle import fp
from oracle.check import bf16_within_1ulp
from oracle.layer import Spec, op_rope_qkv
from synth import attention_case, normal_bf16
from tests._attn import make_cache
from tests._gpu import bf16, bits, f32, i32, same_bits, say

pytestmark = pytest.mark.gpu

HQ, HKV, HD = 32, 8, 128


def _qkv(T, f32_in, strided, seed, hq=HQ, hkv=HKV):
    """Fused projection rows [T, (Hq + 2 Hkv) D] as a device tensor, optionally a view with
    a row stride off the vector width."""
    width = (hq + 2 * hkv) * HD
    pad = 4 if strided else 0
    if f32_in:
        x = (np.random.default_rng(seed).standard_normal((T, width + pad)) * 2).astype(np.float32)
        t = f32(x)
        ref = x[:, :width].astype(np.float64)
    else:
        xb = normal_bf16((T, width + pad), 0.0, 2.0, 91, seed)
        t = bf16(xb)
        ref = fp.bf16_to_f64(xb[:, :width])
    return t[:, :width], ref


@pytest.mark.parametrize("L,ql,ps,qkv_f32,q_f32,strided", [
    ([1400, 37, 3000, 1], [1, 1, 1, 1], 16, False, False, False),      # decode: split path
    ([300, 2049], [300, 1100], 16, False, False, True),                # prefill walk (> 1024 tokens)
    ([700, 260], [200, 260], 64, True, True, False),                   # suffix on a cached prefix
    ([5, 17, 33, 256], [5, 1, 33, 2], 256, False, True, True),
    ([513, 1024, 1025], [1, 1, 1], 32, True, False, True),
])
def test_fused_equals_unfused(lib, L, ql, ps, qkv_f32, q_f32, strided):
    _fused_equals_unfused(lib, L, ql, ps, qkv_f32, q_f32, strided, HQ, HKV)


def test_fused_equals_unfused_many_heads(lib):
    # 64 query + 2 x 8 kv heads: more items per token than two per thread (the kernel's
    # preloaded ones), so the rest go through its trailing loop
    _fused_equals_unfused(lib, [900, 40, 1], [3, 40, 1], 16, False, False, False, 64, 8)


def _fused_equals_unfused(lib, L, ql, ps, qkv_f32, q_f32, strided, hq, hkv):
    say("rope + kv write", L, ql, ps, "fp32 qkv" if qkv_f32 else "bf16 qkv", "fp32 q" if q_f32 else "bf16 q",
        hq, hkv)
    T = sum(ql)
    case = attention_case(L, ql, hq, hkv, HD, cfg=92)
    kc_a, vc_a, bt = make_cache(case, ps, [l - q for l, q in zip(L, ql)], cfg=93)
    kc_b, vc_b = kc_a.clone(), vc_a.clone()
    qkv, qkv64 = _qkv(T, qkv_f32, strided, T + ps, hq, hkv)
    pos = np.concatenate([np.arange(l - q, l) for l, q in zip(L, ql)]).astype(np.int32)
    qsl = np.concatenate([[0], np.cumsum(ql)]).astype(np.int32)
    qd = torch.float32 if q_f32 else torch.bfloat16
    BT, SL, QSL = i32(bt), i32(L), i32(qsl)
    scale = 1.0 / np.sqrt(HD)
    # unfused: RoPE into q, k, v tensors; the attention call writes k and v into the pages
    q_a, k_a, v_a = lib.bi_rope_qkv(qkv, i32(pos), hq, hkv, HD, 10000.0, q_dtype=qd)
    out_a = lib.bi_attention(q_a, k_a, v_a, kc_a, vc_a, BT, SL, QSL, max_seq_len=max(L), scale=scale)
    # fused: RoPE writes q and the pages; the attention call only reads
    q_b = lib.bi_rope_kv_write(qkv, kc_b, vc_b, BT, SL, QSL, hq, 10000.0, q_dtype=qd)
    out_b = lib.bi_attention(q_b, None, None, kc_b, vc_b, BT, SL, QSL, max_seq_len=max(L), scale=scale)
    torch.cuda.synchronize()
    assert same_bits(q_a, q_b)
    assert torch.equal(kc_a.view(torch.int16), kc_b.view(torch.int16))
    assert torch.equal(vc_a.view(torch.int16), vc_b.view(torch.int16))
    assert same_bits(out_a, out_b)
    if T <= 1024:   # the no-allocation form takes the in-cache call too
        out_c = lib.bi_attention_noalloc(q_b, None, None, kc_b, vc_b, BT, SL, QSL, max_seq_len=max(L),
                                         scale=scale)
        assert same_bits(out_c, out_b)
    # the fused queries against the oracle's RoPE (1 bf16 ulp at output scale; fp32 q
    # rounds to the bf16 call's q)
    q64, _, _ = op_rope_qkv(qkv64, pos, Spec(n_q_heads=hq, n_kv_heads=hkv, head_dim=HD))
    qbf = q_b.to(torch.bfloat16) if q_f32 else q_b
    r = bf16_within_1ulp(bits(qbf), q64)
    assert r["ok"], r
