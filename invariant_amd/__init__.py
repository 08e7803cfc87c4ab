"""Python binding of libbi (batch-invariant LLM-forward reductions, MI355X / gfx950).

Argument marshalling only: every function below turns torch tensors into device
pointers, sizes and the current HIP stream, calls the C entry point of the same name
(declared in include/bi.h) and raises BIError on a negative status.  torch provides
device memory and streams; all arithmetic runs in the library's HIP kernels.  There is
no fallback: if libbi.so is missing, ``load()`` raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libbi.so")

BI_BF16, BI_F32 = 1, 2
BI_B_KN, BI_B_NK, BI_B_TILED = 0, 1, 2

_c = ctypes
_P, _I64, _I32, _F32, _F64, _SZ = _c.c_void_p, _c.c_int64, _c.c_int32, _c.c_float, _c.c_double, _c.c_size_t

_SIGS = {
    "bi_get_config": (_c.c_int, [_P]),
    "bi_gemm_tile": (_c.c_int, [_I64, _I64, _I64, _c.c_int, _P, _P, _P]),
    "bi_status_string": (_c.c_char_p, [_c.c_int]),
    "bi_rmsnorm": (_c.c_int, [_P, _P, _P, _I64, _I64, _I64, _I64, _F32, _c.c_int, _c.c_int, _P]),
    "bi_gemm": (_c.c_int, [_P, _P, _P, _I64, _I64, _I64, _I64, _I64, _I64, _c.c_int, _c.c_int, _c.c_int, _P]),
    "bi_gemm_splitk_workspace_bytes": (_SZ, [_I64, _I64, _I64]),
    "bi_gemm_splitk": (_c.c_int, [_P, _P, _P, _I64, _I64, _I64, _I64, _I64, _I64, _c.c_int, _P, _SZ, _P]),
    "bi_gemm_fixed_split_workspace_bytes": (_SZ, [_I64, _I64, _I64, _I64]),
    "bi_gemm_fixed_split": (_c.c_int, [_P, _P, _P, _I64, _I64, _I64, _I64, _I64, _I64, _c.c_int, _I64, _P,
                                       _SZ, _P]),
    "bi_attention_workspace_bytes": (_SZ, [_I64, _I32, _I32, _I64]),
    "bi_attention": (_c.c_int, [_P, _c.c_int, _P, _P, _P, _P, _P, _P, _P, _I32, _I64, _I32, _I32, _I32,
                                _I32, _I32, _I64, _F32, _P, _c.c_int, _P, _SZ, _P]),
    "bi_attention_noalloc": (_c.c_int, [_P, _c.c_int, _P, _P, _P, _P, _P, _P, _P, _I32, _I64, _I32, _I32,
                                        _I32, _I32, _I32, _I64, _F32, _P, _c.c_int, _P]),
    "bi_attention_batchdep_split": (_c.c_int, [_P, _c.c_int, _P, _P, _P, _P, _P, _P, _P, _I32, _I64, _I32,
                                               _I32, _I32, _I32, _I32, _I64, _I64, _F32, _P, _c.c_int,
                                               _P, _SZ, _P]),
    "bi_logsoftmax_argmax": (_c.c_int, [_P, _I64, _I64, _I64, _P, _P, _P]),
    "bi_embedding": (_c.c_int, [_P, _P, _c.c_int, _P, _I64, _I64, _I64, _c.c_int, _P]),
    "bi_rope_qkv": (_c.c_int, [_P, _I64, _c.c_int, _P, _P, _c.c_int, _P, _P, _I64, _I32, _I32, _I32, _F64,
                               _P]),
    "bi_rope_kv_write": (_c.c_int, [_P, _I64, _c.c_int, _P, _c.c_int, _P, _P, _P, _P, _P, _I32, _I64, _I32,
                                    _I32, _I32, _I32, _I32, _F64, _P]),
    "bi_swiglu": (_c.c_int, [_P, _I64, _P, _I64, _I64, _P]),
    "bi_gemm_swiglu": (_c.c_int, [_P, _P, _P, _I64, _I64, _I64, _I64, _I64, _I64, _c.c_int, _P]),
    "bi_pack_b_bytes": (_SZ, [_I64, _I64]),
    "bi_pack_b": (_c.c_int, [_P, _I64, _I64, _I64, _P, _P]),
    "bi_add_rmsnorm": (_c.c_int, [_P, _P, _P, _c.c_int, _P, _P, _c.c_int, _I64, _I64, _c.c_float, _P]),
    "bi_add_rmsnorm_gemm": (_c.c_int, [_P, _P, _P, _P, _c.c_float, _P, _P, _I64, _I64, _I64, _I64, _I64,
                                       _c.c_int, _c.c_int, _P]),
    "bi_add_rmsnorm_gemm_swiglu": (_c.c_int, [_P, _P, _P, _P, _c.c_float, _P, _P, _I64, _I64, _I64, _I64,
                                              _I64, _c.c_int, _P]),
    "bi_residual_add": (_c.c_int, [_P, _c.c_int, _P, _c.c_int, _P, _c.c_int, _I64, _P]),
}
EXPORTS = tuple(_SIGS)


class BIConfig(ctypes.Structure):
    _fields_ = [(n, _I32) for n in (
        "version", "tree_max_lanes", "wave_size", "gemm_tile_m", "gemm_tile_n", "gemm_tile_k",
        "gemm_mfma_m", "gemm_mfma_n", "gemm_mfma_k", "attn_chunk", "attn_max_group",
        "gemm_big_tile_m", "gemm_big_tile_n", "attn_merge_group")]


class BIError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        super().__init__(f"{fn} returned {status} ({status_string(status)})")


_LIB = None


def load(path: str | None = None):
    """Open libbi.so (built by ``python -m invariant_amd.build``); raise if absent."""
    global _LIB
    if _LIB is not None:
        return _LIB
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is not built: run `python -m invariant_amd.build` first")
    lib = ctypes.CDLL(p)
    for name, (res, args) in _SIGS.items():
        f = getattr(lib, name)
        f.restype, f.argtypes = res, args
    _LIB = lib
    return lib


def status_string(status: int) -> str:
    return load().bi_status_string(int(status)).decode()


def get_config() -> dict:
    cfg = BIConfig()
    st = load().bi_get_config(ctypes.byref(cfg))
    if st:
        raise BIError("bi_get_config", st)
    return {n: getattr(cfg, n) for n, _ in BIConfig._fields_}


def _check(fn, st):
    if st != 0:
        raise BIError(fn, st)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(t):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _code(dtype):
    if dtype == torch.bfloat16:
        return BI_BF16
    if dtype == torch.float32:
        return BI_F32
    raise TypeError(f"unsupported dtype {dtype}")


def _ld(t):
    if t.dim() != 2 or (t.stride(1) != 1 and t.shape[1] > 1):
        raise ValueError("expected a 2-D tensor with unit column stride")
    if t.shape[0] > 1 or t.stride(0) >= t.shape[1]:
        return max(t.stride(0), 1)
    return max(t.shape[1], 1)      # one row whose stride torch does not pin down


# ----------------------------------------------------------------------------- calls
def bi_rmsnorm(x, gamma, eps: float, out=None, out_dtype=torch.bfloat16):
    M, D = x.shape
    if out is None:
        out = torch.empty((M, D), dtype=out_dtype, device=x.device)
    _check("bi_rmsnorm", load().bi_rmsnorm(_ptr(x), _ptr(gamma), _ptr(out), M, D, _ld(x), _ld(out),
                                            float(eps), _code(x.dtype), _code(out.dtype), _stream(x)))
    return out


def bi_gemm(a, b, out=None, b_layout: int = BI_B_NK, out_dtype=torch.bfloat16, n=None):
    """C = a @ b^T for b_layout BI_B_NK (b is [N, K]), C = a @ b for BI_B_KN (b is [K, N]);
    BI_B_TILED: b is bi_pack_b of an [N, K] B (N = n, default 16 x its row blocks)."""
    M, K = a.shape
    if b_layout == BI_B_TILED:
        N = n if n is not None else b.shape[0] * 16
        _check_packed("bi_gemm", b, N, K)
        ldb = 0
    else:
        N = b.shape[0] if b_layout == BI_B_NK else b.shape[1]
        ldb = _ld(b)
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=a.device)
    _check("bi_gemm", load().bi_gemm(_ptr(a), _ptr(b), _ptr(out), M, N, K, _ld(a), ldb, _ld(out),
                                      b_layout, _code(a.dtype), _code(out.dtype), _stream(a)))
    return out


def _check_packed(fn, b, N, K):
    """The kernels read ceil(N/16) x ceil(K/32) whole 1 KB tiles of a packed B: refuse a
    tensor of another shape rather than read past it."""
    want = ((N + 15) // 16, (K + 31) // 32, 64, 8)
    if tuple(b.shape) != want or b.dtype != torch.bfloat16 or not b.is_contiguous():
        raise ValueError(f"{fn}: packed B must be a contiguous bf16 tensor of shape {want} "
                         f"(bi_pack_b of an [N, K] B), got {tuple(b.shape)} {b.dtype}")


def bi_pack_b(b):
    """B [N, K] bf16 in the tiled layout of BI_B_TILED: [ceil(N/16), ceil(K/32), 64, 8]."""
    N, K = b.shape
    out = torch.empty(((N + 15) // 16, (K + 31) // 32, 64, 8), dtype=torch.bfloat16, device=b.device)
    _check("bi_pack_b", load().bi_pack_b(_ptr(b), N, K, _ld(b), _ptr(out), _stream(b)))
    return out


def bi_gemm_tile(M: int, N: int, K: int, a_dtype=torch.bfloat16) -> tuple:
    """(rows, columns, LDS ring stages) of the workgroup tile bi_gemm uses for M x N."""
    tm, tn, st = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    _check("bi_gemm_tile", load().bi_gemm_tile(M, N, K, _code(a_dtype), ctypes.byref(tm),
                                                ctypes.byref(tn), ctypes.byref(st)))
    return tm.value, tn.value, st.value


def bi_gemm_splitk(a, b, out=None, out_dtype=torch.bfloat16, workspace=None):
    M, K = a.shape
    N = b.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=a.device)
    need = load().bi_gemm_splitk_workspace_bytes(M, N, K)
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=a.device)
    _check("bi_gemm_splitk", load().bi_gemm_splitk(
        _ptr(a), _ptr(b), _ptr(out), M, N, K, _ld(a), _ld(b), _ld(out), _code(out.dtype),
        _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(a)))
    return out


def bi_gemm_fixed_split(a, b, k_slice: int, out=None, out_dtype=torch.bfloat16, workspace=None):
    """C = a b^T with K cut into slices of k_slice columns at absolute offsets, whatever M is
    (a [M, K], b [N, K] bf16)."""
    M, K = a.shape
    N = b.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=a.device)
    need = load().bi_gemm_fixed_split_workspace_bytes(M, N, K, k_slice)
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=a.device)
    _check("bi_gemm_fixed_split", load().bi_gemm_fixed_split(
        _ptr(a), _ptr(b), _ptr(out), M, N, K, _ld(a), _ld(b), _ld(out), _code(out.dtype), int(k_slice),
        _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(a)))
    return out


def bi_attention_workspace_bytes(num_tokens, num_q_heads, head_dim, max_seq_len) -> int:
    return int(load().bi_attention_workspace_bytes(num_tokens, num_q_heads, head_dim, max_seq_len))


def bi_attention(q, k_new, v_new, k_cache, v_cache, block_table, seq_lens, query_start_loc,
                 max_seq_len: int, scale: float, out=None, out_dtype=torch.bfloat16, workspace=None):
    """q [T, Hq, D], k_new/v_new [T, Hkv, D] bf16 (both None: the new keys and values are in
    the cache already, written by bi_rope_kv_write); k_cache [P, Hkv, D/8, page, 8];
    v_cache [P, Hkv, D, page]; block_table [B, max_pages] int32; seq_lens [B] int32;
    query_start_loc [B + 1] int32 (all on the device)."""
    T, Hq, D = q.shape
    Hkv = k_cache.shape[1]
    page = v_cache.shape[3]
    B, max_pages = block_table.shape
    if out is None:
        out = torch.empty((T, Hq, D), dtype=out_dtype, device=q.device)
    need = bi_attention_workspace_bytes(T, Hq, D, max_seq_len)
    if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    wsz = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("bi_attention", load().bi_attention(
        _ptr(q), _code(q.dtype), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
        _ptr(seq_lens), _ptr(query_start_loc), B, T, Hq, Hkv, D, page, max_pages, int(max_seq_len),
        float(scale), _ptr(out), _code(out.dtype), _ptr(workspace), wsz, _stream(q)))
    return out


def bi_attention_noalloc(q, k_new, v_new, k_cache, v_cache, block_table, seq_lens, query_start_loc,
                         max_seq_len: int, scale: float, out=None, out_dtype=torch.bfloat16):
    """bi_attention with the library's own per-device scratch instead of a workspace (no
    device allocation inside the call; pass `out` to allocate nothing at all)."""
    T, Hq, D = q.shape
    Hkv = k_cache.shape[1]
    page = v_cache.shape[3]
    B, max_pages = block_table.shape
    if out is None:
        out = torch.empty((T, Hq, D), dtype=out_dtype, device=q.device)
    _check("bi_attention_noalloc", load().bi_attention_noalloc(
        _ptr(q), _code(q.dtype), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
        _ptr(seq_lens), _ptr(query_start_loc), B, T, Hq, Hkv, D, page, max_pages, int(max_seq_len),
        float(scale), _ptr(out), _code(out.dtype), _stream(q)))
    return out


def bi_attention_batchdep_split(q, k_new, v_new, k_cache, v_cache, block_table, seq_lens,
                                query_start_loc, max_seq_len: int, total_chunks: int, scale: float,
                                out=None, out_dtype=torch.bfloat16, workspace=None):
    """Comparison variant (not batch-invariant), same layouts as bi_attention."""
    T, Hq, D = q.shape
    Hkv = k_cache.shape[1]
    page = v_cache.shape[3]
    B, max_pages = block_table.shape
    if out is None:
        out = torch.empty((T, Hq, D), dtype=out_dtype, device=q.device)
    need = bi_attention_workspace_bytes(T, Hq, D, max_seq_len)
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    _check("bi_attention_batchdep_split", load().bi_attention_batchdep_split(
        _ptr(q), _code(q.dtype), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
        _ptr(seq_lens), _ptr(query_start_loc), B, T, Hq, Hkv, D, page, max_pages, int(max_seq_len),
        int(total_chunks), float(scale), _ptr(out), _code(out.dtype), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(q)))
    return out


def bi_logsoftmax_argmax(logits, logprobs=None, argmax=None, want_logprobs: bool = True):
    M, V = logits.shape
    ld = _ld(logits)
    if argmax is None:
        argmax = torch.empty((M,), dtype=torch.int32, device=logits.device)
    if logprobs is None and want_logprobs:
        # the call writes logprobs with the row stride of logits
        logprobs = torch.empty_strided((M, V), (ld, 1), dtype=logits.dtype, device=logits.device)
    elif logprobs is not None and (tuple(logprobs.shape) != (M, V) or _ld(logprobs) != ld):
        raise ValueError("logprobs must have the shape and row stride of logits")
    _check("bi_logsoftmax_argmax", load().bi_logsoftmax_argmax(
        _ptr(logits), M, V, ld, _ptr(logprobs), _ptr(argmax), _stream(logits)))
    return logprobs, argmax


def bi_embedding(ids, table, out=None, out_dtype=torch.bfloat16):
    """out[t] = table[ids[t]] (rows of a bf16 or fp32 table, ids int32 on the device)."""
    T = ids.shape[0]
    V, D = table.shape
    if out is None:
        out = torch.empty((T, D), dtype=out_dtype, device=table.device)
    _check("bi_embedding", load().bi_embedding(_ptr(ids), _ptr(table), _code(table.dtype), _ptr(out),
                                                T, D, V, _code(out.dtype), _stream(table)))
    return out


def bi_rope_qkv(qkv, positions, num_q_heads, num_kv_heads, head_dim, base=10000.0,
                q=None, k=None, v=None, q_dtype=torch.bfloat16):
    T = qkv.shape[0]
    dev = qkv.device
    q = q if q is not None else torch.empty((T, num_q_heads, head_dim), dtype=q_dtype, device=dev)
    k = k if k is not None else torch.empty((T, num_kv_heads, head_dim), dtype=torch.bfloat16, device=dev)
    v = v if v is not None else torch.empty((T, num_kv_heads, head_dim), dtype=torch.bfloat16, device=dev)
    _check("bi_rope_qkv", load().bi_rope_qkv(_ptr(qkv), _ld(qkv), _code(qkv.dtype), _ptr(positions),
                                              _ptr(q), _code(q.dtype), _ptr(k), _ptr(v), T, num_q_heads,
                                              num_kv_heads, head_dim, float(base), _stream(qkv)))
    return q, k, v


def bi_rope_kv_write(qkv, k_cache, v_cache, block_table, seq_lens, query_start_loc, num_q_heads,
                     base=10000.0, q=None, q_dtype=torch.bfloat16):
    """bi_rope_qkv fused with bi_attention's cache write: returns q [T, Hq, D]; the rotated
    keys and the values go into k_cache / v_cache at each new token's slot (cache
    positions from seq_lens and query_start_loc).  Follow with bi_attention(q, None, None,
    ...)."""
    T = qkv.shape[0]
    Hkv, D, page = k_cache.shape[1], v_cache.shape[2], v_cache.shape[3]
    B, max_pages = block_table.shape
    if qkv.shape[1] != (num_q_heads + 2 * Hkv) * D:
        raise ValueError(f"bi_rope_kv_write: qkv rows hold {qkv.shape[1]} values, not "
                         f"(num_q_heads + 2 Hkv) D = {(num_q_heads + 2 * Hkv) * D}")
    q = q if q is not None else torch.empty((T, num_q_heads, D), dtype=q_dtype, device=qkv.device)
    if tuple(q.shape) != (T, num_q_heads, D) or not q.is_contiguous():
        raise ValueError(f"bi_rope_kv_write: q must be a contiguous [{T}, {num_q_heads}, {D}] tensor")
    _check("bi_rope_kv_write", load().bi_rope_kv_write(
        _ptr(qkv), _ld(qkv), _code(qkv.dtype), _ptr(q), _code(q.dtype), _ptr(k_cache), _ptr(v_cache),
        _ptr(block_table), _ptr(seq_lens), _ptr(query_start_loc), B, T, num_q_heads, Hkv, D, page,
        max_pages, float(base), _stream(qkv)))
    return q


def bi_swiglu(gu, out=None):
    T, F2 = gu.shape
    F = F2 // 2
    if out is None:
        out = torch.empty((T, F), dtype=torch.bfloat16, device=gu.device)
    _check("bi_swiglu", load().bi_swiglu(_ptr(gu), _ld(gu), _ptr(out), T, F, _stream(gu)))
    return out


def interleave_gate_up(w):
    """[2F, K] gate-then-up weight -> the 16-row interleave bi_gemm_swiglu takes."""
    F2, K = w.shape
    return w.view(2, F2 // 32, 16, K).permute(1, 0, 2, 3).reshape(F2, K).contiguous()


def bi_gemm_swiglu(a, w_interleaved, out=None, w_layout: int = BI_B_NK):
    """swiglu(a @ W^T) with W given as interleave_gate_up(W) (out [M, F] bf16); w_layout
    BI_B_TILED: bi_pack_b(interleave_gate_up(W))."""
    M, K = a.shape
    if w_layout == BI_B_TILED:
        F = w_interleaved.shape[0] * 16 // 2
        _check_packed("bi_gemm_swiglu", w_interleaved, 2 * F, K)
        ldw = 0
    else:
        F = w_interleaved.shape[0] // 2
        ldw = _ld(w_interleaved)
    if out is None:
        out = torch.empty((M, F), dtype=torch.bfloat16, device=a.device)
    _check("bi_gemm_swiglu", load().bi_gemm_swiglu(_ptr(a), _ptr(w_interleaved), _ptr(out), M, F, K,
                                                    _ld(a), ldw, _ld(out), w_layout, _stream(a)))
    return out


def bi_residual_add(a, b, out=None, out_dtype=None):
    if out is None:
        out = torch.empty(a.shape, dtype=out_dtype or a.dtype, device=a.device)
    _check("bi_residual_add", load().bi_residual_add(_ptr(a), _code(a.dtype), _ptr(b), _code(b.dtype),
                                                      _ptr(out), _code(out.dtype), a.numel(), _stream(a)))
    return out


def _norm_gemm_operands(fn, a, b, sum_out, w, w_layout, n_out, K):
    M = a.shape[0]
    if sum_out is None:
        sum_out = torch.empty_like(a)
    for t in (a, b, sum_out):
        if t.shape != (M, K) or not t.is_contiguous() or t.dtype != torch.bfloat16:
            raise ValueError(f"{fn}: a, b and the sum must be contiguous bf16 [M, K]")
    if w_layout == BI_B_TILED:
        _check_packed(fn, w, n_out, K)
        return sum_out, 0
    return sum_out, _ld(w)


def bi_add_rmsnorm_gemm(a, b, gamma, eps: float, w, w_layout: int = BI_B_NK, n=None,
                        out_dtype=torch.bfloat16, sum_out=None, out=None):
    """(s, C): s = a + b and C = rmsnorm(s) @ W^T in one call, the bits of bi_add_rmsnorm
    followed by bi_gemm (at most 4 rows of contiguous bf16 a, b; W [N, K], or with
    BI_B_TILED its bi_pack_b copy and N = n)."""
    M, K = a.shape
    N = (n if n is not None else w.shape[0] * 16) if w_layout == BI_B_TILED else w.shape[0]
    sum_out, ldw = _norm_gemm_operands("bi_add_rmsnorm_gemm", a, b, sum_out, w, w_layout, N, K)
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=a.device)
    _check("bi_add_rmsnorm_gemm", load().bi_add_rmsnorm_gemm(
        _ptr(a), _ptr(b), _ptr(sum_out), _ptr(gamma), float(eps), _ptr(w), _ptr(out), M, N, K, ldw,
        _ld(out), w_layout, _code(out.dtype), _stream(a)))
    return sum_out, out


def bi_add_rmsnorm_gemm_swiglu(a, b, gamma, eps: float, w_interleaved, w_layout: int = BI_B_NK,
                               sum_out=None, out=None):
    """(s, m): s = a + b and m = swiglu(rmsnorm(s) @ W^T) with W as interleave_gate_up(W) (or
    its bi_pack_b copy), the bits of bi_add_rmsnorm followed by bi_gemm_swiglu (at most 4
    rows)."""
    M, K = a.shape
    F = w_interleaved.shape[0] * (16 if w_layout == BI_B_TILED else 1) // 2
    sum_out, ldw = _norm_gemm_operands("bi_add_rmsnorm_gemm_swiglu", a, b, sum_out, w_interleaved,
                                       w_layout, 2 * F, K)
    if out is None:
        out = torch.empty((M, F), dtype=torch.bfloat16, device=a.device)
    _check("bi_add_rmsnorm_gemm_swiglu", load().bi_add_rmsnorm_gemm_swiglu(
        _ptr(a), _ptr(b), _ptr(sum_out), _ptr(gamma), float(eps), _ptr(w_interleaved), _ptr(out), M, F,
        K, ldw, _ld(out), w_layout, _stream(a)))
    return sum_out, out


def bi_add_rmsnorm(a, b, gamma, eps: float, sum_out=None, out=None, out_dtype=torch.bfloat16):
    """(a + b, rmsnorm(a + b)) in one pass; a and b [M, D] contiguous of one dtype."""
    M, D = a.shape
    if sum_out is None:
        sum_out = torch.empty_like(a)
    if out is None:
        out = torch.empty((M, D), dtype=out_dtype, device=a.device)
    for t in (a, b, sum_out, out):
        if t.shape != (M, D) or not t.is_contiguous():
            raise ValueError("bi_add_rmsnorm: operands must be contiguous [M, D]")
    if b.dtype != a.dtype or sum_out.dtype != a.dtype:
        raise ValueError("bi_add_rmsnorm: a, b and the sum share one dtype")
    _check("bi_add_rmsnorm", load().bi_add_rmsnorm(_ptr(a), _ptr(b), _ptr(sum_out), _code(a.dtype), _ptr(gamma),
                                                    _ptr(out), _code(out.dtype), M, D, float(eps), _stream(a)))
    return sum_out, out
