"""Paged-cache plumbing for the attention GPU tests (layout of include/bi.h):
k_cache [page][kv head][D/8][slot'][8] with slot' = slot with bits 2 and 3 swapped,
v_cache [page][kv head][D][slot]."""
import numpy as np
import torch

from synth import paged_layout
from tests._gpu import bf16, i32

NAN_BF16 = 0x7FC0


def k_slot(s):
    """Physical slot of logical slot s inside a K page (bits 2 and 3 swapped)."""
    s = np.asarray(s)
    return (s & ~12) | ((s & 4) << 1) | ((s & 8) >> 1)


def k_logical(kc, pages, n):
    """Read keys 0..n-1 back from K pages into [n, Hkv, D] (logical order)."""
    P, hkv, dg, ps, e = kc.shape
    pos = np.arange(n)
    pg = torch.from_numpy(np.asarray(pages)[pos // ps].astype(np.int64)).cuda()
    sl = torch.from_numpy(k_slot(pos % ps).astype(np.int64)).cuda()
    return kc[pg, :, :, sl, :].reshape(n, hkv, dg * e)


def make_cache(case, page_size, prior, cfg=77, extra_pages=5, hkv=None, d=None):
    """Pages for every sequence (shuffled), the first prior[b] positions written, every
    other slot holding NaN so that a read of an unwritten slot would show."""
    L = case["seq_lens"]
    k0 = case["k"][0]
    hkv = hkv or k0.shape[1]
    d = d or k0.shape[2]
    bt, total = paged_layout(L, page_size, cfg, 7, extra_pages)
    kc = torch.full((total, hkv, d // 8, page_size, 8), NAN_BF16, dtype=torch.int16, device="cuda")
    vc = torch.full((total, hkv, d, page_size), NAN_BF16, dtype=torch.int16, device="cuda")
    kc, vc = kc.view(torch.bfloat16), vc.view(torch.bfloat16)
    for b, n in enumerate(prior):
        if n == 0:
            continue
        pos = np.arange(n)
        pages = torch.from_numpy(bt[b, pos // page_size].astype(np.int64)).cuda()
        slots = torch.from_numpy((pos % page_size).astype(np.int64)).cuda()
        kslots = torch.from_numpy(k_slot(pos % page_size).astype(np.int64)).cuda()
        kc[pages, :, :, kslots, :] = bf16(case["k"][b][:n]).reshape(n, hkv, d // 8, 8)
        vc[pages, :, :, slots] = bf16(case["v"][b][:n])
    return kc, vc, bt


def run(lib, case, kc, vc, bt, out_dtype=torch.bfloat16, scale=None):
    L, ql = case["seq_lens"], case["q_lens"]
    q = np.concatenate([case["q"][b] for b in range(len(L))])
    kn = np.concatenate([case["k"][b][L[b] - ql[b]:L[b]] for b in range(len(L))])
    vn = np.concatenate([case["v"][b][L[b] - ql[b]:L[b]] for b in range(len(L))])
    qsl = np.concatenate([[0], np.cumsum(ql)]).astype(np.int32)
    d = q.shape[-1]
    out = lib.bi_attention(bf16(q), bf16(kn), bf16(vn), kc, vc, i32(bt), i32(L), i32(qsl),
                           max_seq_len=max(L), scale=scale or 1.0 / np.sqrt(d), out_dtype=out_dtype)
    return out, qsl
