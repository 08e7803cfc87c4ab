"""Mistral-7B-shaped composition of the batch-invariant calls: paged KV cache, decoder
layer, full model and greedy decoding.

Orchestration only: every arithmetic step is one of the library's entry points; torch
provides device memory and the stream.  Sources:
  * "Defeating nondeterminism in LLM inference": a request's output must not depend on
    the server's batch (batch invariance); the KV cache and page table are updated
    before the attention kernel (bi_rope_kv_write does it with the rotation, or, when a
    layer is traced, bi_attention does it first from k and v tensors); chunked prefill
    must give the same numbers as an unsplit prefill.
  * "Does the same LLM give different outputs on different GPUs? Why?": greedy decoding
    of a Mistral-7B model on a ~1400-token prompt, token probabilities from the
    normalised scores.
  * arXiv abstract on cross-vendor mismatch: upcasting to FP32 except the MLPs, which stay
    in BF16 ("fp32 variant" below).

Layer (pre-norm, SwiGLU):
  x  = rmsnorm(h);  q, k, v = rope(split(x Wqkv^T));  a = attention(q, k, v | cache)
  h2 = h + a Wo^T;  x2 = rmsnorm(h2);  out = h2 + (silu(x2 Wg^T) * (x2 Wu^T)) Wd^T
bf16 model: every activation is stored in bf16.  fp32 variant: the residual stream, the
attention-side norm, projections, q and the attention output are fp32 (fp32 x bf16 products
through the exact three-way split in bi_gemm and bi_attention); the MLP (its norm output,
gate/up, SwiGLU, down) stays bf16; the KV cache stays bf16 (storage, as the weights are);
logits are fp32 in both.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

from . import (bi_attention, bi_attention_workspace_bytes, bi_embedding, bi_gemm,
               bi_logsoftmax_argmax, bi_residual_add, bi_rmsnorm, bi_rope_kv_write, bi_rope_qkv,
               bi_swiglu, bi_gemm_swiglu, interleave_gate_up, bi_add_rmsnorm, bi_pack_b,
               bi_add_rmsnorm_gemm, bi_add_rmsnorm_gemm_swiglu, BI_B_NK, BI_B_TILED)

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
    return with_derived_weights(w)


# Copies of a layer's weights in other layouts, made from its [N, K] matrices: the gate/up
# rows interleaved in blocks of 16 for the fused GEMM + SwiGLU call (wgate_up keeps the
# gate-then-up order the reference computations read), and every projection tiled
# (bi_pack_b) for calls of a few rows -- the same bits, contiguous kilobyte loads.
DERIVED = ("wgate_up_i", "wqkv_t", "wo_t", "wgate_up_t", "wdown_t")


def with_derived_weights(w: dict) -> dict:
    w["wgate_up_i"] = interleave_gate_up(w["wgate_up"])
    w["wgate_up_t"] = bi_pack_b(w["wgate_up_i"])
    for k in ("wqkv", "wo", "wdown"):
        w[k + "_t"] = bi_pack_b(w[k])
    return w


def random_model(dims: Dims, seed: int, device="cuda", sd=0.02):
    """Random-init weights of the given shape (linear and embedding ~ N(0, sd), norm
    gammas ~ N(1, 0.02)), drawn by a seeded device generator."""
    gen = torch.Generator(device=device).manual_seed(seed)
    return _with_tiled_head(dict(
        embed=_normal((dims.vocab, dims.hidden), 0.0, sd, gen, device),
        layers=[random_layer(dims, gen, device, sd) for _ in range(dims.n_layers)],
        final_norm=_normal((dims.hidden,), 1.0, 0.02, gen, device),
        lm_head=_normal((dims.vocab, dims.hidden), 0.0, sd, gen, device),
    ))


def _with_tiled_head(model):
    model["lm_head_t"] = bi_pack_b(model["lm_head"])
    return model


_CUS = {}


def _cus(dev) -> int:
    if dev not in _CUS:
        _CUS[dev] = torch.cuda.get_device_properties(dev).multi_processor_count
    return _CUS[dev]


def _tiled_ok(a: torch.Tensor, n: int) -> bool:
    """Whether an [M, K] x [N, K]^T call reads the tiled copy of its weight.  A tiled B
    serves the few-row kernel (include/bi.h, BI_B_TILED: at most 64 rows of bf16 A, K a
    multiple of 8 and at least 1024); among those calls it is the faster operand except
    (measured on MI355X with the weights streamed from HBM, Mistral-7B shapes, same bits
    either way) above 32 rows on grids of more 32-column blocks than CUs, where the [N, K]
    weight goes to the 128 x 128 tiles (gate/up, LM head at 49 rows: 51 and 61 us against
    68 and 71), and up to 16 rows when one 16-column block per wave leaves at most one wave
    per CU (O and down at 16 rows: 10.1 and 29.7 us against 11.3 and 31.7)."""
    m, k = a.shape
    if m > 64 or k % 8 or k < 1024 or a.dtype != BF16:
        return False
    cus = _cus(a.device)
    if m > 32:
        return (n + 31) // 32 <= cus
    return m > 16 or (n + 15) // 16 > cus


def _linear(x: torch.Tensor, w: dict, name: str, out_dtype) -> torch.Tensor:
    """x @ w[name]^T, from the tiled copy w[name + "_t"] where there is one and it pays."""
    n = w[name].shape[0]
    if name + "_t" in w and _tiled_ok(x, n):
        return bi_gemm(x, w[name + "_t"], b_layout=BI_B_TILED, n=n, out_dtype=out_dtype)
    return bi_gemm(x, w[name], out_dtype=out_dtype)


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


def _norm_fused(h, dims: Dims, fp32_variant: bool, trace) -> bool:
    """Whether the layer's residual adds and RMSNorms run inside the projections that read
    them (bi_add_rmsnorm_gemm, bi_add_rmsnorm_gemm_swiglu; bf16 residual stream, hidden size a
    multiple of 8 in [1024, 4096]; untraced layers, whose normalised rows are never kept).
    The calls take up to 4 rows, but every workgroup replays the rows' norm before its first
    product, which pays for the saved launch only at one row (measured on MI355X at the
    Mistral-7B shapes, kernel time: QKV 14.1 us fused against 11.4 + 4.3, gate/up 45.9
    against 42.8 + 4.3; at 4 rows 20.8 against 11.8 + 4.6)."""
    return (trace is None and not fp32_variant and h.shape[0] == 1 and h.dtype == BF16
            and dims.hidden % 8 == 0 and 1024 <= dims.hidden <= 4096)


def _norm_linear(a, d, w, norm: str, name: str, dims: Dims):
    """(a + d, rmsnorm(a + d) @ w[name]^T) in one launch, from the tiled copy where it pays."""
    n = w[name].shape[0]
    if name + "_t" in w and _tiled_ok(a, n):
        return bi_add_rmsnorm_gemm(a, d, w[norm], dims.eps, w[name + "_t"], w_layout=BI_B_TILED, n=n)
    return bi_add_rmsnorm_gemm(a, d, w[norm], dims.eps, w[name])


def decoder_layer(w, h, batch: Batch, k_cache, v_cache, dims: Dims, fp32_variant=False,
                  x=None, next_norm=None, trace=None, d=None, defer=False):
    """One layer on the residual stream h.  x, if given, is rmsnorm(h) with this layer's
    attention norm (the previous layer computed it with its residual add).  With next_norm the
    layer returns (h_out, rmsnorm(h_out) with next_norm), else h_out.  d, if given, is the
    previous layer's down projection not yet added: the layer's input is h + d.  With defer
    the layer leaves its own last residual add to the next layer and returns (h2, dn).  An
    untraced bf16 row runs each residual add and RMSNorm inside the projection that reads it
    (bi_add_rmsnorm_gemm, bi_add_rmsnorm_gemm_swiglu).  Every path gives the same
    bits as the separate calls.  trace, if a dict, receives the layer's intermediate
    tensors by name (h, x, qkv, q, k, v, attn, o, h2, x2, mlp, dn, out, next_x); a traced
    layer keeps k and v as tensors (bi_rope_qkv, then bi_attention writes them into the
    pages), an untraced one rotates straight into the pages (bi_rope_kv_write): the same
    bits either way."""
    T = h.shape[0]
    act = F32 if fp32_variant else BF16
    fused = _norm_fused(h, dims, fp32_variant, trace)
    if d is not None and fused:
        h, qkv = _norm_linear(h, d, w, "attn_norm", "wqkv", dims)
    else:
        if d is not None:
            h, x = bi_add_rmsnorm(h, d, w["attn_norm"], dims.eps, out_dtype=act)
        elif x is None:
            x = bi_rmsnorm(h, w["attn_norm"], dims.eps, out_dtype=act)
        qkv = _linear(x, w, "wqkv", act)
    if trace is None:   # RoPE writes the rotated keys and the values straight into the pages
        q = bi_rope_kv_write(qkv, k_cache, v_cache, batch.block_table, batch.seq_lens, batch.qsl,
                             dims.n_q_heads, dims.rope_base, q_dtype=act)
        k = v = None
    else:               # the same bits through k and v tensors, which the trace keeps
        q, k, v = bi_rope_qkv(qkv, batch.positions, dims.n_q_heads, dims.n_kv_heads, dims.head_dim,
                              dims.rope_base, q_dtype=act)
    a = bi_attention(q, k, v, k_cache, v_cache, batch.block_table, batch.seq_lens, batch.qsl,
                     batch.max_seq_len, 1.0 / float(np.sqrt(dims.head_dim)), out_dtype=act,
                     workspace=batch.workspace)
    o = _linear(a.view(T, dims.n_q_heads * dims.head_dim), w, "wo", act)
    x2 = None
    if fused and "wgate_up_i" in w:   # add, norm, gate/up and SwiGLU in one launch
        tiled = _tiled_ok(h, w["wgate_up"].shape[0])
        h2, m = bi_add_rmsnorm_gemm_swiglu(h, o, w["ffn_norm"], dims.eps,
                                           w["wgate_up_t"] if tiled else w["wgate_up_i"],
                                           w_layout=BI_B_TILED if tiled else BI_B_NK)
    else:
        if _fusable(h, o, dims):
            h2, x2 = bi_add_rmsnorm(h, o, w["ffn_norm"], dims.eps, out_dtype=BF16)
        else:
            h2 = bi_residual_add(h, o, out_dtype=act)
            x2 = bi_rmsnorm(h2, w["ffn_norm"], dims.eps, out_dtype=BF16)
        if "wgate_up_t" in w and _tiled_ok(x2, w["wgate_up"].shape[0]):   # a few rows: the tiled copy
            m = bi_gemm_swiglu(x2, w["wgate_up_t"], w_layout=BI_B_TILED)
        elif "wgate_up_i" in w:   # fused: == bi_swiglu(bi_gemm(x2, wgate_up)) bit for bit
            m = bi_gemm_swiglu(x2, w["wgate_up_i"])
        else:
            m = bi_swiglu(bi_gemm(x2, w["wgate_up"]))
    dn = _linear(m, w, "wdown", BF16)
    if defer:
        return h2, dn
    if next_norm is None:
        res = bi_residual_add(h2, dn, out_dtype=act)
        h3, x3 = res, None
    elif _fusable(h2, dn, dims):
        res = h3, x3 = bi_add_rmsnorm(h2, dn, next_norm, dims.eps, out_dtype=act)
    else:
        h3 = bi_residual_add(h2, dn, out_dtype=act)
        res = h3, x3 = h3, bi_rmsnorm(h3, next_norm, dims.eps, out_dtype=act)
    if trace is not None:
        trace.update(h=h, x=x, qkv=qkv, q=q, k=k, v=v, attn=a, o=o, h2=h2, x2=x2, mlp=m, dn=dn,
                     out=h3, next_x=x3)
    return res


def forward(model, batch: Batch, cache: PagedKVCache, dims: Dims, fp32_variant=False,
            on_layer=None):
    """The layers over one ragged call.  on_layer(li, trace) is called after each layer with
    its intermediate tensors (see decoder_layer); trace["emb"] holds the embedding rows."""
    act = F32 if fp32_variant else BF16
    h = bi_embedding(batch.tokens, model["embed"], out_dtype=act)
    layers = model["layers"]
    x = d = None
    for li, w in enumerate(layers):
        tr = None if on_layer is None else ({"emb": h} if li == 0 else {})
        if li + 1 < len(layers) and _norm_fused(h, dims, fp32_variant, tr):
            # one row: the down projection's residual add goes, with the next layer's
            # attention norm, into that layer's QKV projection
            h, d = decoder_layer(w, h, batch, cache.k[li], cache.v[li], dims, fp32_variant,
                                 x=x, trace=tr, d=d, defer=True)
            x = None
        elif li + 1 < len(layers):   # the next layer's attention norm rides on this residual add
            h, x = decoder_layer(w, h, batch, cache.k[li], cache.v[li], dims, fp32_variant,
                                 x=x, next_norm=layers[li + 1]["attn_norm"], trace=tr, d=d)
            d = None
        else:
            h = decoder_layer(w, h, batch, cache.k[li], cache.v[li], dims, fp32_variant, x=x,
                              trace=tr, d=d)
        if on_layer is not None:
            on_layer(li, tr)
    return h


def head(model, h, rows: torch.Tensor, dims: Dims, fp32_variant=False):
    """Final norm, LM head (fp32 logits) and the greedy pick for the given rows of h."""
    act = F32 if fp32_variant else BF16
    hl = bi_embedding(rows, h, out_dtype=h.dtype)
    x = bi_rmsnorm(hl, model["final_norm"], dims.eps, out_dtype=act)
    logits = _linear(x, model, "lm_head", F32)
    _, ids = bi_logsoftmax_argmax(logits, want_logprobs=False)
    return logits, ids


def greedy_generate(model, prompts, n_new: int, cache: PagedKVCache, dims: Dims,
                    fp32_variant=False, max_chunk_tokens: int = 16384, keep_logits=None,
                    sid_base: int = 0, timings: dict | None = None):
    """Greedy decoding of a ragged batch.  The prompts are prefilled in chunks of at most
    max_chunk_tokens tokens (a prompt may be split across chunks), then every sequence
    decodes one token per step.  Returns (tokens [B, n_new] int32 numpy, logits dict
    {b: [n_new, V] fp32 tensor} for b in keep_logits).  timings, if a dict, receives the
    wall-clock seconds of the prefill (up to the first tokens on the host) and of the decode
    steps after it (up to the last tokens on the host)."""
    import time
    t_start = time.perf_counter()
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
    t_prefill = time.perf_counter()   # (the first tokens are on the host: the work is done)
    # decode: every sequence's pages for the whole generation are reserved up front, so the
    # block table stays fixed; each step's argmax is the next step's token on the device and
    # the positions and lengths advance in place, so the host issues step after step without
    # waiting for one (the token ids come back once, at the end)
    dev = torch.device("cuda")
    lens = [len(p) for p in prompts]
    final = [n + n_new - 1 for n in lens]
    for s, f in zip(sids, final):
        cache.reserve(s, f)
    msl = max(final)
    ws = bi_attention_workspace_bytes(B, dims.n_q_heads, dims.head_dim, msl)
    pos = torch.tensor(lens, dtype=torch.int32, device=dev)
    batch = Batch(tokens=torch.tensor(first, dtype=torch.int32, device=dev), positions=pos,
                  block_table=torch.from_numpy(cache.table(sids)).to(dev), seq_lens=pos + 1,
                  qsl=torch.arange(B + 1, dtype=torch.int32, device=dev), max_seq_len=msl,
                  workspace=torch.empty(ws, dtype=torch.uint8, device=dev) if ws else None)
    rows = torch.arange(B, dtype=torch.int32, device=dev)
    keep_list = sorted(keep)
    keep_idx = torch.tensor(keep_list, dtype=torch.int64, device=dev)
    ids_all, kept = [batch.tokens], []
    for step in range(1, n_new):
        h = forward(model, batch, cache, dims, fp32_variant)
        lg, ids = head(model, h, rows, dims, fp32_variant)
        ids_all.append(ids)
        if keep_list:   # the kept rows in one gather per step
            kept.append(lg.index_select(0, keep_idx))
        batch.tokens = ids
        batch.positions.add_(1)
        batch.seq_lens.add_(1)
    if kept:
        dec = torch.stack(kept, dim=1)   # [kept sequences, decode steps, V]
        for r, i in enumerate(keep_list):
            logits_out[i].extend(dec[r].unbind(0))
    tokens = torch.stack(ids_all, dim=1).cpu().numpy().astype(np.int32)
    if timings is not None:
        timings.update(prefill_s=t_prefill - t_start, decode_s=time.perf_counter() - t_prefill,
                       decode_steps=n_new - 1)
    for s in sids:
        cache.release(s)
    return tokens, {i: torch.stack(v) for i, v in logits_out.items()}
