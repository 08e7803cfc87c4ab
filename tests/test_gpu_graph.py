"""The hot-path calls captured in one HIP graph: every replay gives the eager bits.

The library launches only kernels on the caller's stream (no allocation, no memset, no
synchronisation), so a caller may capture a pass of the path and replay it.  Each replay
here follows eager work and a synchronisation, and all outputs are zeroed before it, so a
replay that skipped or corrupted a write would show.
"""
import numpy as np
import pytest
import torch

from synth import attention_case, gemm_inputs, rmsnorm_linear_inputs
from tests._attn import make_cache
from tests._gpu import bf16, f32, i32, same_bits, say

pytestmark = pytest.mark.gpu


def test_graph_replays_equal_eager(lib):
    say("graph: rmsnorm + gemm (tiles and few rows) + attention decode + log-softmax")
    x, gamma, w = rmsnorm_linear_inputs(300, 4096, 1024)
    X, G, W = bf16(x), bf16(gamma), bf16(w)
    a, b = gemm_inputs(8, 2048, 1024, cfg=41)
    A8, B8 = bf16(a), bf16(np.ascontiguousarray(b.T))
    L = [700, 1, 260, 1500]
    case = attention_case(L, [1] * len(L), cfg=42)
    kc, vc, bt = make_cache(case, 16, [l - 1 for l in L], cfg=43)
    q = bf16(np.concatenate([case["q"][i] for i in range(len(L))]))
    kn = bf16(np.concatenate([case["k"][i][L[i] - 1:L[i]] for i in range(len(L))]))
    vn = bf16(np.concatenate([case["v"][i][L[i] - 1:L[i]] for i in range(len(L))]))
    qsl = i32(np.arange(len(L) + 1))
    ws = torch.empty(lib.bi_attention_workspace_bytes(len(L), 32, 128, max(L)), dtype=torch.uint8, device="cuda")
    logits = f32((np.random.default_rng(44).standard_normal((4, 32000)) * 2).astype(np.float32))
    out = dict(y=torch.empty_like(X), c=torch.empty((300, 1024), dtype=torch.bfloat16, device="cuda"),
               c8=torch.empty((8, 2048), dtype=torch.bfloat16, device="cuda"),
               o=torch.empty((len(L), 32, 128), dtype=torch.bfloat16, device="cuda"),
               lp=torch.empty((4, 32000), dtype=torch.float32, device="cuda"),
               am=torch.empty((4,), dtype=torch.int32, device="cuda"))

    def step():
        lib.bi_rmsnorm(X, G, 1e-5, out=out["y"])
        lib.bi_gemm(out["y"], W, out=out["c"])
        lib.bi_gemm(A8, B8, out=out["c8"])
        lib.bi_attention(q, kn, vn, kc, vc, BT, SL, qsl, max_seq_len=max(L),
                         scale=1.0 / np.sqrt(128.0), out=out["o"], workspace=ws)
        lib.bi_logsoftmax_argmax(logits, logprobs=out["lp"], argmax=out["am"])

    BT, SL = i32(bt), i32(np.asarray(L, np.int32))
    step()
    torch.cuda.synchronize()
    eager = {k: v.clone() for k, v in out.items()}
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(4):
        for v in out.values():
            v.zero_()
        lib.bi_gemm(A8, B8)          # unrelated eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k in out:
            assert same_bits(out[k], eager[k]), (rep, k)
