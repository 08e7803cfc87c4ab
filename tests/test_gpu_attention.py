"""bi_attention on the GPU: within 1 bf16 ulp of the fp64 oracle at the scale of each
(token, head) output, and bitwise invariant to the batch, the path (split-KV decode or
prefill walk), the physical pages and the position of a sequence in the batch.

Cited: "Defeating nondeterminism in LLM inference", section on batch-invariant attention
(update the KV cache and page table before the kernel; a token must reduce in the same
order whether 0 or p tokens are cached; split-KV for decode).
"""
import numpy as np
import pytest
import torch

from oracle.attention import attention_case_f64
from oracle.check import bf16_within_1ulp, f32_within_rel
from synth import attention_case, ragged_lengths
from tests._attn import k_logical, make_cache, run
from tests._gpu import bits, host, same_bits, say

pytestmark = pytest.mark.gpu


def _check_vs_oracle(case, out, qsl, which=None):
    ref = attention_case_f64(case, which)
    o = bits(out)
    for b, r in enumerate(ref):
        idx = range(case["q_lens"][b]) if which is None else which.get(b, [])
        for j, i in enumerate(idx):
            got = o[qsl[b] + i]
            res = bf16_within_1ulp(got, r[j])
            assert res["ok"], (b, i, res)


@pytest.mark.parametrize("hq,hkv", [(32, 8), (8, 8), (16, 1), (8, 4)])
def test_prefill_small_vs_oracle(lib, hq, hkv):
    say("attention prefill", hq, hkv)
    L = [1, 37, 256, 300]
    case = attention_case(L, L, hq, hkv, 128, cfg=40, salt=hq)
    kc, vc, bt = make_cache(case, 16, [0] * len(L))
    out, qsl = run(lib, case, kc, vc, bt)
    _check_vs_oracle(case, out, qsl)


def test_decode_vs_oracle_and_prefill_bitwise(lib):
    L = [255, 256, 257, 513, 1400, 3000]
    pre = attention_case(L, L, cfg=41)                       # 5681 tokens: prefill walk
    kc, vc, bt = make_cache(pre, 16, [0] * len(L))
    out_p, qsl_p = run(lib, pre, kc, vc, bt)
    dec = attention_case(L, [1] * len(L), cfg=41)            # same sequences, last token new
    kc2, vc2, bt2 = make_cache(dec, 16, [l - 1 for l in L], cfg=78)
    out_d, qsl_d = run(lib, dec, kc2, vc2, bt2)
    for b, l in enumerate(L):
        assert same_bits(out_d[b], out_p[qsl_p[b] + l - 1]), b
    _check_vs_oracle(dec, out_d, qsl_d)
    _check_vs_oracle(pre, out_p, qsl_p, which={b: [0, l // 2, l - 1] for b, l in enumerate(L)})
    # the K/V the prefill wrote into its pages are the logical sequence
    pages = torch.from_numpy(bt[5, :3].astype(np.int64)).cuda()
    got = k_logical(kc, bt[5], 48)
    assert np.array_equal(bits(got), pre["k"][5][:48])
    gotv = vc[pages].permute(0, 3, 1, 2).reshape(48, 8, 128)
    assert np.array_equal(bits(gotv), pre["v"][5][:48])


def test_batch_position_page_invariance(lib):
    L = ragged_lengths(8, 300, 2500, 42, 0)
    case = attention_case(L, [1] * 8, cfg=42)
    kc, vc, bt = make_cache(case, 16, [l - 1 for l in L])
    out, _ = run(lib, case, kc, vc, bt)
    for b in (0, 5):
        one = {k: [case[k][b]] for k in ("seq_lens", "q_lens", "k", "v", "q")}
        for cfg in (79, 80):                                  # two different page permutations
            kc1, vc1, bt1 = make_cache(one, 16, [L[b] - 1], cfg=cfg)
            o1, _ = run(lib, one, kc1, vc1, bt1)
            assert same_bits(o1[0], out[b])
    rev = {k: case[k][::-1] for k in ("seq_lens", "q_lens", "k", "v", "q")}
    kcr, vcr, btr = make_cache(rev, 16, [l - 1 for l in rev["seq_lens"]], cfg=81)
    outr, _ = run(lib, rev, kcr, vcr, btr)
    assert same_bits(outr.flip(0), out)
    # page size 32 and 256 give the same bits (chunks are logical)
    for ps in (32, 256):
        kcp, vcp, btp = make_cache(case, ps, [l - 1 for l in L], cfg=82)
        op, _ = run(lib, case, kcp, vcp, btp)
        assert same_bits(op, out), ps


def test_split_work_list_edges(lib):
    # decode batches of many short or mixed sequences: the split kernel's work list (token,
    # chunk, kv head) is walked by a persistent grid with look-ahead, so every workgroup
    # runs past the end of its list, and the smallest call has fewer items than workgroups.
    # The large batches take 4-chunk work units and a single sequence one-chunk units (the
    # combine kernel then merges the chunks of each group): both give the same bits.
    rng = np.random.default_rng(44)
    for B, lo, hi, hq, hkv in [(97, 1, 1500, 32, 8), (3, 1, 20, 8, 1), (40, 250, 260, 16, 1)]:
        say("split work list", B, lo, hi, hq, hkv)
        L = [int(x) for x in rng.integers(lo, hi + 1, B)]
        dec = attention_case(L, [1] * B, n_q_heads=hq, n_kv_heads=hkv, cfg=44)
        kc, vc, bt = make_cache(dec, 16, [l - 1 for l in L], cfg=84)
        out, qsl = run(lib, dec, kc, vc, bt)
        _check_vs_oracle(dec, out, qsl)
        for b in (0, B // 2, B - 1):   # each sequence alone gives the same bits
            one = {k: [dec[k][b]] for k in ("seq_lens", "q_lens", "k", "v", "q")}
            kc1, vc1, bt1 = make_cache(one, 16, [L[b] - 1], cfg=85)
            o1, _ = run(lib, one, kc1, vc1, bt1)
            assert same_bits(o1[0], out[b]), (B, b)


def test_chunked_prefill_matches_full_prefill(lib):
    L = 1100
    full = attention_case([L], [L], cfg=43)
    kc, vc, bt = make_cache(full, 16, [0])
    out_full, _ = run(lib, full, kc, vc, bt)
    # the same prompt in pieces of 300, 1, 512, 287 new tokens
    kc2, vc2, bt2 = make_cache(full, 16, [0], cfg=83)
    start = 0
    for piece in (300, 1, 512, 287):
        part = attention_case([start + piece], [piece], cfg=43)
        o, _ = run(lib, part, kc2, vc2, bt2)
        assert same_bits(o, out_full[start:start + piece]), piece
        start += piece


def test_paged_decode_batch64_long_contexts(lib):
    B = 64
    L = ragged_lengths(B, 1400, 32768, 4, 0)
    case = attention_case(L, [1] * B, cfg=4)
    kc, vc, bt = make_cache(case, 16, [l - 1 for l in L])
    out, qsl = run(lib, case, kc, vc, bt)
    _check_vs_oracle(case, out, qsl, which={b: [0] for b in range(0, B, 9)})
    for m in (1, 7, 33):
        sub = {k: case[k][:m] for k in ("seq_lens", "q_lens", "k", "v", "q")}
        o, _ = run(lib, sub, kc, vc, bt[:m].copy())
        assert same_bits(o, out[:m]), m
    of, _ = run(lib, case, kc, vc, bt, out_dtype=torch.float32)
    ref = attention_case_f64(case, {0: [0]})[0][0]
    assert f32_within_rel(host(of[0]), ref)["ok"]


def test_decode_equals_prefill_long_contexts(lib):
    L = [4000, 9000]
    pre = attention_case(L, L, cfg=44)
    kc, vc, bt = make_cache(pre, 16, [0, 0])
    out_p, qsl_p = run(lib, pre, kc, vc, bt)
    dec = attention_case(L, [1, 1], cfg=44)
    kc2, vc2, bt2 = make_cache(dec, 16, [l - 1 for l in L], cfg=84)
    out_d, _ = run(lib, dec, kc2, vc2, bt2)
    for b, l in enumerate(L):
        assert same_bits(out_d[b], out_p[qsl_p[b] + l - 1])


def test_decode_equals_prefill_at_32k_boundaries(lib):
    # decode == prefill bitwise across the last 1024-key group boundaries of the 32k context
    # (16383/16384/16385 and 32767/32768 keys: a group of four chunks just full, or one key
    # into the next), and the decode rows within 1 ulp of the oracle from the same calls
    L = [16383, 16384, 16385, 32767, 32768]
    say("prefill", sum(L), "tokens")
    pre = attention_case(L, L, cfg=47)
    kc, vc, bt = make_cache(pre, 16, [0] * len(L))
    out_p, qsl_p = run(lib, pre, kc, vc, bt)
    say("decode")
    dec = attention_case(L, [1] * len(L), cfg=47)
    kc2, vc2, bt2 = make_cache(dec, 16, [l - 1 for l in L], cfg=86)
    out_d, qsl_d = run(lib, dec, kc2, vc2, bt2)
    for b, l in enumerate(L):
        assert same_bits(out_d[b], out_p[qsl_p[b] + l - 1]), l
    _check_vs_oracle(dec, out_d, qsl_d, which={b: [0] for b in range(len(L))})


def test_fp32_q(lib):
    # q in fp32 (the FP32-activation variant): each value split exactly into bf16 hi + mid + lo
    # for the scores.  (1) With bf16-representable q values the split adds exact zeros, so the
    # bits equal the bf16-q call's; (2) with full fp32 q, decode == prefill bitwise on both
    # paths and the rows are within 1e-3 (fp32 out) and 1 ulp (bf16 out) of the oracle at
    # output scale, which holds q at full precision
    from oracle.attention import attention_values_f64
    from oracle import fp as F
    from tests._gpu import bf16, f32, i32
    L = [700, 1500, 2100]
    dec = attention_case(L, [1, 1, 1], cfg=51)
    kc, vc, bt = make_cache(dec, 16, [l - 1 for l in L])
    q_b = np.concatenate(dec["q"])
    kn = np.concatenate([dec["k"][b][L[b] - 1:L[b]] for b in range(3)])
    vn = np.concatenate([dec["v"][b][L[b] - 1:L[b]] for b in range(3)])
    args = (bf16(kn), bf16(vn), kc, vc, i32(bt), i32(L), i32(np.arange(4)))
    ref16 = lib.bi_attention(bf16(q_b), *args, max_seq_len=max(L), scale=1 / np.sqrt(128.0))
    got = lib.bi_attention(bf16(q_b).float(), *args, max_seq_len=max(L), scale=1 / np.sqrt(128.0))
    assert same_bits(got, ref16)
    # full fp32 q, the same per position in prefill and decode
    rng = np.random.default_rng(51)
    qf = {b: rng.standard_normal((L[b], 32, 128)).astype(np.float32) for b in range(3)}
    pre = attention_case(L, L, cfg=51)
    kcp, vcp, btp = make_cache(pre, 16, [0, 0, 0], cfg=87)
    qp = np.concatenate([qf[b] for b in range(3)])
    knp = np.concatenate(pre["k"])
    vnp = np.concatenate(pre["v"])
    qsl = np.concatenate([[0], np.cumsum(L)]).astype(np.int32)
    outp = lib.bi_attention(f32(qp), bf16(knp), bf16(vnp), kcp, vcp, i32(btp), i32(L), i32(qsl),
                            max_seq_len=max(L), scale=1 / np.sqrt(128.0), out_dtype=torch.float32)
    qd = np.stack([qf[b][-1] for b in range(3)])
    for out_dtype in (torch.float32, torch.bfloat16):
        outd = lib.bi_attention(f32(qd), *args, max_seq_len=max(L), scale=1 / np.sqrt(128.0),
                                out_dtype=out_dtype)
        for b in range(3):
            ref = attention_values_f64(qd[b:b + 1].astype(np.float64), F.bf16_to_f64(dec["k"][b]),
                                       F.bf16_to_f64(dec["v"][b]), [L[b] - 1])[0]
            if out_dtype == torch.float32:
                assert same_bits(outd[b], outp[qsl[b] + L[b] - 1]), b
                r = f32_within_rel(host(outd[b]), ref)
            else:
                r = bf16_within_1ulp(bits(outd[b]), ref)
            assert r["ok"], (b, out_dtype, r)
    # a prefill row checked directly too (the walk path)
    mid = 1000
    ref = attention_values_f64(qf[1][mid:mid + 1].astype(np.float64), F.bf16_to_f64(pre["k"][1][:mid + 1]),
                               F.bf16_to_f64(pre["v"][1][:mid + 1]), [mid])[0]
    assert f32_within_rel(host(outp[qsl[1] + mid]), ref)["ok"]


def test_batchdep_split_variant_correct_but_not_invariant(lib):
    B = 32
    L = ragged_lengths(B, 1400, 8000, 46, 0)
    case = attention_case(L, [1] * B, cfg=46)
    kc, vc, bt = make_cache(case, 16, [l - 1 for l in L])
    inv, qsl = run(lib, case, kc, vc, bt)
    q = np.concatenate(case["q"])
    kn = np.concatenate([case["k"][b][L[b] - 1:L[b]] for b in range(B)])
    vn = np.concatenate([case["v"][b][L[b] - 1:L[b]] for b in range(B)])
    total = int(sum((int(l) - 1) // 256 + 1 for l in L))
    from tests._gpu import bf16, i32
    var = lib.bi_attention_batchdep_split(bf16(q), bf16(kn), bf16(vn), kc, vc, i32(bt), i32(L),
                                          i32(np.arange(B + 1)), int(max(L)), total,
                                          1.0 / np.sqrt(128))
    _check_vs_oracle(case, var, qsl, which={b: [0] for b in (0, 7, 31)})
    # alone, a sequence gets one chunk per split (the invariant association) ...
    one = {k: [case[k][0]] for k in ("seq_lens", "q_lens", "k", "v", "q")}
    kc1, vc1, bt1 = make_cache(one, 16, [int(L[0]) - 1], cfg=85)
    alone = lib.bi_attention_batchdep_split(bf16(q[:1]), bf16(kn[:1]), bf16(vn[:1]), kc1, vc1,
                                            i32(bt1), i32(L[:1]), i32(np.arange(2)), int(L[0]),
                                            (int(L[0]) - 1) // 256 + 1, 1.0 / np.sqrt(128))
    assert same_bits(alone[0], inv[0])
    # ... inside the batch its chunks are grouped, so its bits move with the batch
    n_diff = sum(int(not same_bits(var[b], inv[b])) for b in range(B))
    say("batch-dependent split: sequences whose bits changed", n_diff, "of", B)
    assert n_diff > 0
