"""Op-by-op parity of a traced decoder layer (invariant_amd.model.decoder_layer with a trace
dict) against the oracle: every oracle operation is fed the GPU's OWN stored inputs to that
operation, so each op keeps the bar it has on its own ("Defeating nondeterminism in LLM
inference", section on making kernels batch-invariant: the layer is its operations):

  RMSNorm (plain or fused with the residual add)  bit-exact (tree replay)
  residual add                                    bit-exact (one rounding of an exact sum)
  embedding gather, v split                       bit-exact
  GEMMs (QKV, O, gate/up, down), attention        within 1 bf16 ulp at output scale;
                                                  fp32 outputs within 1e-3 at output scale
  RoPE, SwiGLU                                    within 1 bf16 ulp of the fp64 formula
                                                  rounded once
  fused gate/up + SwiGLU                          bitwise bi_swiglu(bi_gemm(...)), and
                                                  inside the interval the projection's
                                                  1-ulp bar allows (oracle.check)
"""
import numpy as np
import torch

from invariant_amd.model import DERIVED
from oracle import fp
from oracle.check import bf16_within_1ulp, bits_equal, f32_within_rel, swiglu_interval_within
from oracle.layer import Spec, op_attention, op_gemm, op_rmsnorm, op_rope_qkv, store, swiglu_f64


def values(t: torch.Tensor) -> np.ndarray:
    """Stored values of a bf16 or fp32 tensor as float64 (exact)."""
    t = t.detach().contiguous()
    if t.dtype == torch.bfloat16:
        return fp.bf16_to_f64(t.view(torch.int16).cpu().numpy().view(np.uint16))
    return t.float().cpu().numpy().astype(np.float64)


def dtype_of(t: torch.Tensor) -> str:
    return "bf16" if t.dtype == torch.bfloat16 else "f32"


def _same(got64, want64, dtype):
    """Bit equality of stored values (as the stored type's bits)."""
    if dtype == "bf16":
        return bits_equal(fp.f64_to_bf16(got64), fp.f64_to_bf16(want64))
    return bits_equal(np.asarray(got64, np.float32), np.asarray(want64, np.float32))


def _near(got64, ref64, dtype, axis=-1):
    if dtype == "bf16":
        return bf16_within_1ulp(fp.f64_to_bf16(got64), ref64, axis=axis)
    return f32_within_rel(got64, ref64, 1e-3, axis=axis)


def host_weights(w: dict) -> dict:
    """Layer weights (device bf16 tensors) as bf16 bit arrays (the re-laid-out copies of the
    gate/up matrix left out)."""
    return {k: v.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
            for k, v in w.items() if k not in DERIVED}


def take(trace: dict, rows) -> dict:
    """The rows of every [T, ...] tensor of a layer trace, on the host as stored values, with
    their dtypes."""
    idx = torch.as_tensor(np.asarray(rows, dtype=np.int64), device="cuda")
    out = {}
    for k, t in trace.items():
        if isinstance(t, torch.Tensor):
            out[k] = (values(t.index_select(0, idx)), dtype_of(t))
    return out


def check_layer(lib, rows_tr: dict, wb: dict, w_dev: dict, positions, kv_ctx, spec: Spec,
                tag: str = "") -> dict:
    """rows_tr: take(trace, rows); wb: host_weights; w_dev: device weights (for the extra
    unfused gate/up GEMM); positions: absolute positions of the rows; kv_ctx(i) -> (K, V)
    stored values [p + 1, Hkv, D] of row i's keys/values 0..p (its own new key last).
    Returns {op: report}; every report has 'ok'."""
    R = {}
    g = lambda k: rows_tr[k][0]
    dt = lambda k: rows_tr[k][1]
    act = spec.act
    n = g("h").shape[0]
    hq, hkv, hd = spec.n_q_heads, spec.n_kv_heads, spec.head_dim
    # attention-side norm
    R["rmsnorm"] = _same(g("x"), op_rmsnorm(g("h"), wb["attn_norm"], spec.eps, dt("h"), dt("x")), dt("x"))
    # fused projection
    R["gemm_qkv"] = _near(g("qkv"), op_gemm(g("x"), wb["wqkv"], dt("x")), dt("qkv"))
    # RoPE + split
    q64, k64, v64 = op_rope_qkv(g("qkv"), positions, spec)
    R["rope_q"] = _near(g("q").reshape(n, hq, hd), q64, dt("q"))
    R["rope_k"] = _near(g("k").reshape(n, hkv, hd), k64, dt("k"))
    R["split_v"] = _same(g("v").reshape(n, hkv, hd), store(v64, dt("v")), dt("v"))
    # attention, row by row over its own context
    q = g("q").reshape(n, hq, hd)
    ref = np.stack([op_attention(q[i:i + 1], *kv_ctx(i), [int(positions[i])])[0] for i in range(n)])
    R["attention"] = _near(g("attn").reshape(n, hq, hd), ref, dt("attn"))
    # output projection, residual add, MLP norm
    R["gemm_o"] = _near(g("o"), op_gemm(g("attn").reshape(n, hq * hd), wb["wo"], dt("attn")), dt("o"))
    R["residual_attn"] = _same(g("h2"), store(g("h") + g("o"), dt("h2")), dt("h2"))
    R["rmsnorm_ffn"] = _same(g("x2"), op_rmsnorm(g("h2"), wb["ffn_norm"], spec.eps, dt("h2"), dt("x2")),
                             dt("x2"))
    # gate/up: the unfused GEMM on the GPU's x2 rows, its SwiGLU, and the fused output
    x2d = torch.from_numpy(fp.f64_to_bf16(g("x2")).view(np.int16)).cuda().view(torch.bfloat16)
    gu_dev = lib.bi_gemm(x2d, w_dev["wgate_up"])
    gu = values(gu_dev)
    gu_ref = op_gemm(g("x2"), wb["wgate_up"], "bf16")
    R["gemm_gate_up"] = _near(gu, gu_ref, "bf16")
    F = gu.shape[1] // 2
    sw_dev = lib.bi_swiglu(gu_dev)
    R["swiglu"] = _near(values(sw_dev), swiglu_f64(gu[:, :F], gu[:, F:]), "bf16")
    R["fused_equals_unfused"] = _same(g("mlp"), values(sw_dev), "bf16")
    R["gemm_swiglu_interval"] = swiglu_interval_within(fp.f64_to_bf16(g("mlp")), gu_ref[:, :F], gu_ref[:, F:])
    # down projection and the residual add
    R["gemm_down"] = _near(g("dn"), op_gemm(g("mlp"), wb["wdown"], "bf16"), dt("dn"))
    R["residual_mlp"] = _same(g("out"), store(g("h2") + g("dn"), dt("out")), dt("out"))
    if rows_tr.get("next_x") is not None and "next_norm" in wb:
        R["rmsnorm_next"] = _same(g("next_x"), op_rmsnorm(g("out"), wb["next_norm"], spec.eps, dt("out"),
                                                         dt("next_x")), dt("next_x"))
    bad = {k: v for k, v in R.items() if not v["ok"]}
    if tag:
        worst = {k: round(v.get("max_ulps", v.get("max_rel", 0.0)), 3) for k, v in R.items()
                 if "max_ulps" in v or "max_rel" in v}
        print(tag, "ops ok" if not bad else f"FAILED {sorted(bad)}", worst, flush=True)
    return R
