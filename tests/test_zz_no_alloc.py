"""bi_attention_noalloc (the attention entry point that allocates nothing: its partials live in
the library's per-device scratch) through the C ABI: bit for bit the output of bi_attention
with a caller workspace, on two calls in a row -- a 16-sequence decode over contexts of up to
32k keys, then a smaller 2-sequence call, which reuses (and overwrites) the same scratch --
and on a prefill long enough to take the walk path (no scratch)."""
import numpy as np
import pytest
import torch

from synth import attention_case, ragged_lengths
from tests._attn import make_cache
from tests._gpu import bf16, i32, same_bits, say

pytestmark = pytest.mark.gpu


def _inputs(case):
    L, ql = case["seq_lens"], case["q_lens"]
    q = np.concatenate([case["q"][b] for b in range(len(L))])
    kn = np.concatenate([case["k"][b][L[b] - ql[b]:L[b]] for b in range(len(L))])
    vn = np.concatenate([case["v"][b][L[b] - ql[b]:L[b]] for b in range(len(L))])
    qsl = np.concatenate([[0], np.cumsum(ql)]).astype(np.int32)
    return bf16(q), bf16(kn), bf16(vn), i32(qsl)


def _compare(lib, case, prior, cfg):
    kc, vc, bt = make_cache(case, 16, prior, cfg=cfg)
    q, kn, vn, qsl = _inputs(case)
    L = case["seq_lens"]
    args = (q, kn, vn, kc, vc, i32(bt), i32(L), qsl)
    for out_dtype in (torch.bfloat16, torch.float32):
        ref = lib.bi_attention(*args, max_seq_len=max(L), scale=1.0 / np.sqrt(128.0), out_dtype=out_dtype)
        out = torch.full_like(ref, float("nan"))
        got = lib.bi_attention_noalloc(*args, max_seq_len=max(L), scale=1.0 / np.sqrt(128.0), out=out)
        torch.cuda.synchronize()
        assert got.data_ptr() == out.data_ptr()
        assert same_bits(got, ref), (case["seq_lens"][:4], out_dtype)


def test_noalloc_equals_workspace_call(lib):
    L = [int(x) for x in ragged_lengths(16, 1400, 32768, 80, 0)]
    say("noalloc: 16-sequence decode, max context", max(L))
    _compare(lib, attention_case(L, [1] * 16, cfg=80), [l - 1 for l in L], cfg=81)
    say("noalloc: 2-sequence decode (smaller, same scratch)")
    L2 = [300, 1500]
    _compare(lib, attention_case(L2, [1, 1], cfg=82), [l - 1 for l in L2], cfg=83)
    say("noalloc: 1100-token prefill (walk path, no scratch)")
    _compare(lib, attention_case([1100], [1100], cfg=84), [0], cfg=85)
