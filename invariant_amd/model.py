"""Mistral-7B-shaped composition of the batch-invariant calls: paged KV cache, decoder
layer, full model and greedy decoding.

Orchestration only: every arithmetic step is one of the library's entry points; torch
provides device memory and the stream.  Sources:
  * "Defeating nondeterminism in LLM inference": a request's output must not depend on
    the server's batch (batch invariance); the KV cache and page table are updated
    before the attention kernel (bi_attention does that first); chunked prefill must
    give the same numbers as an unsplit prefill.
  * "Does the same LLM give different outputs on different GPUs? Why?": greedy decoding
    of a Mistral-7B model on a ~1400-token prompt, token probabilities from the
    normalised scores.
  * arXiv abstract on cross-vendor mismatch: upcasting to FP32 except the MLPs, which stay
    in BF16 ("fp32 variant" below).

Layer (pre-norm, SwiGLU):
  x  = rmsnorm(h);  q, k, v = rope(split(x Wqkv^T));  a = attention(q, k, v | cache)
  h2 = h + a Wo^T;  x2 = rmsnorm(h2);  out = h2 + (silu(x2 Wg^T) * (x2 Wu^T)) Wd^T
bf16 model: every activation is stored in bf16.  fp32 variant: the residual stream, the
attention-side norm, projections and attention output are fp32 (fp32 x bf16-weight
products through bi_gemm's exact three-way split); the MLP (its norm output, gate/up,
SwiGLU, down) stays bf16; the KV cache stays bf16; logits are fp32 in both.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

from . import (bi_attention, bi_attention_workspace_bytes, bi_embedding, bi_gemm,
               bi_logsoftmax_argmax, bi_residual_add, bi_rmsnorm, bi_rope_qkv, bi_swiglu,
               bi_gemm_swiglu, interleave_gate_up, bi_add_rmsnorm)

BF16, F32 = torch.bfloat16, torch.float32


@dataclass
class Dims:
    hidden: int = 4096
    n_q_heads: int = 32
    n_kv_heads: int = 8
    head_dim: int = 128
    ffn: int = 14336
    vocab: int = 32000
    n_layers: int = 32
    eps: float = 1e-5
    rope_base: float = 10000.0


# ------------------------------------------------------------------------- weights
def _normal(shape, mean, sd, gen, device):
    t = torch.randn(shape, generator=gen, device=device, dtype=F32)
    if sd != 1.0:
        t.mul_(sd)
    if mean != 0.0:
        t.add_(mean)
    return t.to(BF16)


def random_layer(dims: Dims, gen, device="cuda", sd=0.02):
    d, hd = dims.hidden, dims.head_dim
    qkv = (dims.n_q_heads + 2 * dims.n_kv_heads) * hd
    w = dict(
        attn_norm=_normal((d,), 1.0, 0.02, gen, device),
        wqkv=_normal((qkv, d), 0.0, sd, gen, device),
        wo=_normal((d, dims.n_q_heads * hd), 0.0, sd, gen, device),
        ffn_norm=_normal((d,), 1.0, 0.02, gen, device),
        wgate_up=_normal((2 * dims.ffn, d), 0.0, sd, gen, device),
        wdown=_normal((d, dims.ffn), 0.0, sd, gen, device),
    )
    # the same gate/up rows interleaved in blocks of 16 for the fused GEMM + SwiGLU call
    # (wgate_up keeps the gate-then-up order the reference computations read)
    w["wgate_up_i"] = interleave_gate_up(w["wgate_up"])
    return w


def random_model(dims: Dims, seed: int, device="cuda", sd=0.02):
    """Random-init weights of the given shape (linear and embedding ~ N(0, sd), norm
    gammas ~ N(1, 0.02)), drawn by a seeded device generator."""
    gen = torch.Generator(device=device).manual_seed(seed)
    return dict(
        embed=_normal((dims.vocab, dims.hidden), 0.0, sd, gen, device),
        layers=[random_layer(dims, gen, device, sd) for _ in range(dims.n_layers)],
        final_norm=_normal((dims.hidden,), 1.0, 0.02, gen, device),
        lm_head=_normal((dims.vocab, dims.hidden), 0.0, sd, gen, device),
    )


# ------------------------------------------------------------------------- KV cache
class PagedKVCache:
    """K/V pages of every layer plus a host-side page allocator.  Pages are handed out
    from a seeded random permutation of the pool, so logical order never matches
    physical order.  Layout per layer: include/bi.h (k [page][kv head][D/8][slot'][8],
    v [page][kv head][D][slot])."""

    def __init__(self, dims: Dims, n_pages: int, page_size: int = 16, device="cuda",
                 seed: int = 0, n_layers: int | None = None):
        nl = dims.n_layers if n_layers is None else n_layers
        hkv, hd = dims.n_kv_heads, dims.head_dim
        self.page_size = page_size
        self.k = torch.zeros((nl, n_pages, hkv, hd // 8, page_size, 8), dtype=BF16, device=device)
        self.v = torch.zeros((nl, n_pages, hkv, hd, page_size), dtype=BF16, device=device)
        self.free = [int(p) for p in np.random.default_rng(seed).permutation(n_pages)]
        self.pages: dict[int, list[int]] = {}

    def reserve(self, sid: int, length: int):
        pages = self.pages.setdefault(sid, [])
        need = -(-length // self.page_size)
        while len(pages) < need:
            if not self.free:
                raise RuntimeError("KV cache out of pages")
            pages.append(self.free.pop())

    def release(self, sid: int):
        self.free.extend(self.pages.pop(sid, []))

    def table(self, sids) -> np.ndarray:
        width = max(1, max(len(self.pages.get(s, [])) for s in sids))
        bt = np.zeros((len(sids), width), dtype=np.int32)
        for i, s in enumerate(sids):
            p = self.pages.get(s, [])
            bt[i, :len(p)] = p
        return bt


@dataclass
class Batch:
    """Device-side metadata of one ragged forward call."""
    tokens: torch.Tensor          # [T] int32
    positions: torch.Tensor       # [T] int32
    block_table: torch.Tensor     # [B, max_pages] int32
    seq_lens: torch.Tensor        # [B] int32 (tokens stored after the call)
    qsl: torch.Tensor             # [B + 1] int32
    max_seq_len: int
    workspace: torch.Tensor | None


def make_batch(cache: PagedKVCache, sids, done, new_tokens, device="cuda", dims: Dims | None = None):
    """sids: sequences in this call; done[i]: tokens already cached for sids[i];
    new_tokens[i]: np.int32 array of its new tokens."""
    dims = dims or Dims()
    seq_lens, toks, pos, qsl = [], [], [], [0]
    for s, d, t in zip(sids, done, new_tokens):
        n = len(t)
        cache.reserve(s, d + n)
        seq_lens.append(d + n)
        toks.append(np.asarray(t, dtype=np.int32))
        pos.append(np.arange(d, d + n, dtype=np.int32))
        qsl.append(qsl[-1] + n)
    T = qsl[-1]
    msl = max(seq_lens)
    ws_bytes = bi_attention_workspace_bytes(T, dims.n_q_heads, dims.head_dim, msl)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(device)
    return Batch(tokens=dev(np.concatenate(toks)), positions=dev(np.concatenate(pos)),
                 block_table=dev(cache.table(sids)), seq_lens=dev(np.asarray(seq_lens, np.int32)),
                 qsl=dev(np.asarray(qsl, np.int32)), max_seq_len=msl,
                 workspace=torch.empty(ws_bytes, dtype=torch.uint8, device=device) if ws_bytes else None)


# ------------------------------------------------------------------------- forward
def _fusable(h, o, dims: Dims):
    """bi_add_rmsnorm takes contiguous rows of one dtype, D a multiple of 8 up to 8192."""
    return dims.hidden % 8 == 0 and dims.hidden <= 8192 and o.dtype == h.dtype


def decoder_layer(w, h, batch: Batch, k_cache, v_cache, dims: Dims, fp32_variant=False,
                  x=None, next_norm=None):
    """One layer on the residual stream h.  x, if given, is rmsnorm(h) with this layer's
    attention norm (the previous layer computed it with its residual add).  With next_norm the
    layer returns (h_out, rmsnorm(h_out) with next_norm), else h_out.  Every path gives the
    same bits as the separate calls."""
    T = h.shape[0]
    act = F32 if fp32_variant else BF16
    if x is None:
        x = bi_rmsnorm(h, w["attn_norm"], dims.eps, out_dtype=act)
    qkv = bi_gemm(x, w["wqkv"], out_dtype=act)
    q, k, v = bi_rope_qkv(qkv, batch.positions, dims.n_q_heads, dims.n_kv_heads, dims.head_dim,
                          dims.rope_base)
    a = bi_attention(q, k, v, k_cache, v_cache, batch.block_table, batch.seq_lens, batch.qsl,
                     batch.max_seq_len, 1.0 / float(np.sqrt(dims.head_dim)), out_dtype=act,
                     workspace=batch.workspace)
    o = bi_gemm(a.view(T, dims.n_q_heads * dims.head_dim), w["wo"], out_dtype=act)
    if _fusable(h, o, dims):
        h2, x2 = bi_add_rmsnorm(h, o, w["ffn_norm"], dims.eps, out_dtype=BF16)
    else:
        h2 = bi_residual_add(h, o, out_dtype=act)
        x2 = bi_rmsnorm(h2, w["ffn_norm"], dims.eps, out_dtype=BF16)
    if "wgate_up_i" in w:   # fused: == bi_swiglu(bi_gemm(x2, wgate_up)) bit for bit
        m = bi_gemm_swiglu(x2, w["wgate_up_i"])
    else:
        m = bi_swiglu(bi_gemm(x2, w["wgate_up"]))
    dn = bi_gemm(m, w["wdown"])
    if next_norm is None:
        return bi_residual_add(h2, dn, out_dtype=act)
    if _fusable(h2, dn, dims):
        return bi_add_rmsnorm(h2, dn, next_norm, dims.eps, out_dtype=act)
    h3 = bi_residual_add(h2, dn, out_dtype=act)
    return h3, bi_rmsnorm(h3, next_norm, dims.eps, out_dtype=act)


def forward(model, batch: Batch, cache: PagedKVCache, dims: Dims, fp32_variant=False):
    act = F32 if fp32_variant else BF16
    h = bi_embedding(batch.tokens, model["embed"], out_dtype=act)
    layers = model["layers"]
    x = None
    for li, w in enumerate(layers):
        if li + 1 < len(layers):   # the next layer's attention norm rides on this residual add
            h, x = decoder_layer(w, h, batch, cache.k[li], cache.v[li], dims, fp32_variant,
                                 x=x, next_norm=layers[li + 1]["attn_norm"])
        else:
            h = decoder_layer(w, h, batch, cache.k[li], cache.v[li], dims, fp32_variant, x=x)
    return h


def head(model, h, rows: torch.Tensor, dims: Dims, fp32_variant=False):
    """Final norm, LM head (fp32 logits) and the greedy pick for the given rows of h."""
    act = F32 if fp32_variant else BF16
    hl = bi_embedding(rows, h, out_dtype=h.dtype)
    x = bi_rmsnorm(hl, model["final_norm"], dims.eps, out_dtype=act)
    logits = bi_gemm(x, model["lm_head"], out_dtype=F32)
    _, ids = bi_logsoftmax_argmax(logits, want_logprobs=False)
    return logits, ids


def greedy_generate(model, prompts, n_new: int, cache: PagedKVCache, dims: Dims,
                    fp32_variant=False, max_chunk_tokens: int = 16384, keep_logits=None,
                    sid_base: int = 0):
    """Greedy decoding of a ragged batch.  The prompts are prefilled in chunks of at most
    max_chunk_tokens tokens (a prompt may be split across chunks), then every sequence
    decodes one token per step.  Returns (tokens [B, n_new] int32 numpy, logits dict
    {b: [n_new, V] fp32 tensor} for b in keep_logits)."""
    B = len(prompts)
    keep = set(range(B)) if keep_logits is None else set(keep_logits)
    sids = [sid_base + i for i in range(B)]
    done = [0] * B
    first = [None] * B
    logits_out = {b: [] for b in keep}
    # chunked ragged prefill
    b = 0
    while b < B:
        budget = max_chunk_tokens
        part_sids, part_done, part_new, part_idx = [], [], [], []
        while b < B and budget > 0:
            rem = len(prompts[b]) - done[b]
            take = min(rem, budget)
            part_sids.append(sids[b]); part_done.append(done[b]); part_idx.append(b)
            part_new.append(np.asarray(prompts[b][done[b]:done[b] + take], dtype=np.int32))
            budget -= take
            done[b] += take
            if done[b] == len(prompts[b]):
                b += 1
        batch = make_batch(cache, part_sids, part_done, part_new, dims=dims)
        h = forward(model, batch, cache, dims, fp32_variant)
        qsl = batch.qsl.cpu().numpy()
        fin = [(j, i) for j, i in enumerate(part_idx) if done[i] == len(prompts[i])]
        if fin:
            rows = torch.tensor([int(qsl[j + 1]) - 1 for j, _ in fin], dtype=torch.int32, device=h.device)
            lg, ids = head(model, h, rows, dims, fp32_variant)
            ids = ids.cpu().numpy()
            for r, (j, i) in enumerate(fin):
                first[i] = int(ids[r])
                if i in keep:
                    logits_out[i].append(lg[r].clone())
        del h
    tokens = np.zeros((B, n_new), dtype=np.int32)
    tokens[:, 0] = first
    cur = list(first)
    lens = [len(p) for p in prompts]
    for step in range(1, n_new):
        batch = make_batch(cache, sids, lens, [np.asarray([t], np.int32) for t in cur], dims=dims)
        h = forward(model, batch, cache, dims, fp32_variant)
        rows = torch.arange(B, dtype=torch.int32, device=h.device)
        lg, ids = head(model, h, rows, dims, fp32_variant)
        ids = ids.cpu().numpy()
        for i in range(B):
            tokens[i, step] = ids[i]
            if i in keep:
                logits_out[i].append(lg[i].clone())
        lens = [l + 1 for l in lens]
        cur = list(ids)
    for s in sids:
        cache.release(s)
    return tokens, {i: torch.stack(v) for i, v in logits_out.items()}
