#!/usr/bin/env python3
"""bench.py -- one pass of the batch-invariant hot path on one MI355X.

A step runs, back to back on one stream, the four reductions of the path at their
headline sizes (one batch of synthetic, Mistral-7B-shaped input):
  a1  bi_rmsnorm            x bf16 [65536, 4096], gamma ~ N(1, 0.02), eps 1e-5
  a2  bi_gemm               bf16 2048 x 2048 x 2048, A, B ~ N(0, 1), fp32 accumulate
  a3  bi_attention decode   64 sequences, context ~ U[1400, 32768], 32 q / 8 kv heads,
                            head_dim 128, page 16 (shuffled pages), one new token each
  a4  bi_logsoftmax_argmax  fp32 logits [64, 32000] (the greedy head of those 64 tokens)
`value` is the step's fraction of the MI355X roofline in percent: the time the step's
algorithmic work needs at peak (HBM 8 TB/s for a1, a3, a4; dense bf16 MFMA 2.5 PFLOP/s
for a2) divided by the measured step time.  Per-row TFLOP/s and GB/s are reported in
`components`; `roofline` describes the dominant call (attention decode).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--gemm-sweep]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

HBM_PEAK = 8.0e12          # bytes/s, MI355X HBM3E
BF16_PEAK = 2.5e15         # flop/s, dense bf16 MFMA
METRIC = "batch-invariant GEMM TFLOP/s + RMSNorm/attn-decode GB/s, % of MI355X peak"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def build_inputs(torch, bi):
    import synth
    dev = "cuda:0"
    g = torch.Generator(device=dev).manual_seed(1234)
    inp = {}
    # a1
    M, D = 65536, 4096
    inp["x"] = torch.randn((M, D), generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
    inp["gamma"] = torch.from_numpy(synth.normal_bf16((D,), 1.0, 0.02, 90, 1).view(np.int16)).to(dev).view(torch.bfloat16)
    # a2
    a, b = synth.gemm_inputs(2048, 2048, 2048, cfg=2)
    inp["A"] = torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
    inp["B_nk"] = torch.from_numpy(np.ascontiguousarray(b.T).view(np.int16)).to(dev).view(torch.bfloat16)
    # a3
    B, hq, hkv, hd, ps = 64, 32, 8, 128, 16
    L = synth.ragged_lengths(B, 1400, 32768, 4, 0)
    bt, total = synth.paged_layout(L, ps, 4, 7, 0)
    inp["L"] = L
    inp["k_cache"] = torch.randn((total, hkv, hd // 8, ps, 8), generator=g, device=dev).to(torch.bfloat16)
    inp["v_cache"] = torch.randn((total, hkv, hd, ps), generator=g, device=dev).to(torch.bfloat16)
    inp["bt"] = torch.from_numpy(bt).to(dev)
    inp["seq_lens"] = torch.from_numpy(L.astype(np.int32)).to(dev)
    inp["qsl"] = torch.arange(B + 1, dtype=torch.int32, device=dev)
    inp["q"] = torch.randn((B, hq, hd), generator=g, device=dev).to(torch.bfloat16)
    inp["k_new"] = torch.randn((B, hkv, hd), generator=g, device=dev).to(torch.bfloat16)
    inp["v_new"] = torch.randn((B, hkv, hd), generator=g, device=dev).to(torch.bfloat16)
    inp["attn_out"] = torch.empty((B, hq, hd), dtype=torch.bfloat16, device=dev)
    ws = bi.bi_attention_workspace_bytes(B, hq, hd, int(L.max()))
    inp["ws"] = torch.empty(ws, dtype=torch.uint8, device=dev)
    # a4
    inp["logits"] = torch.randn((B, 32000), generator=g, device=dev) * 2.0
    # outputs
    inp["y"] = torch.empty((M, D), dtype=torch.bfloat16, device=dev)
    inp["C"] = torch.empty((2048, 2048), dtype=torch.bfloat16, device=dev)
    inp["lp"] = torch.empty((B, 32000), dtype=torch.float32, device=dev)
    inp["am"] = torch.empty((B,), dtype=torch.int32, device=dev)
    torch.cuda.synchronize()
    return inp


def work(inp):
    M, D = inp["x"].shape
    L = inp["L"]
    B, hq, hd = inp["q"].shape
    hkv = inp["k_new"].shape[1]
    V = inp["logits"].shape[1]
    return {
        "rmsnorm": dict(bytes=4 * M * D + 2 * D, flops=0, bound="hbm"),
        "gemm": dict(bytes=3 * 2048 * 2048 * 2, flops=2 * 2048 ** 3, bound="mfma"),
        "attention_decode": dict(
            bytes=int(2 * 2 * hkv * hd * int(L.sum()) + 2 * 2 * B * hq * hd + 2 * 2 * B * hkv * hd),
            flops=int(4 * hq * hd * int(L.sum())), bound="hbm"),
        "logsoftmax_argmax": dict(bytes=8 * B * V + 4 * B, flops=0, bound="hbm"),
    }


def step_ops(bi, inp):
    L = inp["L"]
    return [
        ("rmsnorm", lambda: bi.bi_rmsnorm(inp["x"], inp["gamma"], 1e-5, out=inp["y"])),
        ("gemm", lambda: bi.bi_gemm(inp["A"], inp["B_nk"], out=inp["C"])),
        ("attention_decode", lambda: bi.bi_attention(
            inp["q"], inp["k_new"], inp["v_new"], inp["k_cache"], inp["v_cache"], inp["bt"],
            inp["seq_lens"], inp["qsl"], max_seq_len=int(L.max()), scale=1.0 / np.sqrt(128.0),
            out=inp["attn_out"], workspace=inp["ws"])),
        ("logsoftmax_argmax", lambda: bi.bi_logsoftmax_argmax(inp["logits"], logprobs=inp["lp"],
                                                               argmax=inp["am"])),
    ]


def cpu_baseline(inp, torch, work_d, t_peak_step):
    """Time the oracle, as it stands, on a bounded sample of the same step."""
    import oracle
    from oracle.attention import attention_rows_f64
    from oracle.gemm import gemm_f64
    from oracle.logsoftmax import logsoftmax_argmax
    from oracle.rmsnorm import rmsnorm_tree

    def bits(t):
        return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)

    est = {}
    # a1: 1024 of 65536 rows
    xs = bits(inp["x"][:1024]); g = bits(inp["gamma"])
    t0 = time.perf_counter(); rmsnorm_tree(xs, g, 1e-5); est["rmsnorm"] = (time.perf_counter() - t0) * 64
    # a2: 256 of 2048 rows
    a = bits(inp["A"][:256]); b = bits(inp["B_nk"])
    t0 = time.perf_counter(); gemm_f64(a, b, "nk"); est["gemm"] = (time.perf_counter() - t0) * 8
    # a3: 4 of 64 sequences, gathered from the pages into logical order
    L = inp["L"]; bt = inp["bt"].cpu().numpy(); ps = inp["v_cache"].shape[3]
    sample = [0, 16, 32, 48]
    t_att = 0.0
    for bb in sample:
        n = int(L[bb]); pages = torch.from_numpy(bt[bb, :(n + ps - 1) // ps].astype(np.int64)).cuda()
        pos = np.arange(n)
        kslot = (pos % ps & ~12) | ((pos % ps & 4) << 1) | ((pos % ps & 8) >> 1)
        k = bits(inp["k_cache"][torch.from_numpy(bt[bb, pos // ps].astype(np.int64)).cuda(), :, :,
                                torch.from_numpy(kslot.astype(np.int64)).cuda(), :].reshape(n, 8, 128))
        v = bits(inp["v_cache"][pages].permute(0, 3, 1, 2).reshape(-1, 8, 128)[:n])
        q = bits(inp["q"][bb:bb + 1])
        t0 = time.perf_counter(); attention_rows_f64(q, k, v, [n - 1]); t_att += time.perf_counter() - t0
    frac = sum(int(L[bb]) for bb in sample) / float(L.sum())
    est["attention_decode"] = t_att / frac
    # a4: 16 of 64 rows
    lg = inp["logits"][:16].cpu().numpy()
    t0 = time.perf_counter(); logsoftmax_argmax(lg); est["logsoftmax_argmax"] = (time.perf_counter() - t0) * 4
    total = sum(est.values())
    return {
        "value": 100.0 * t_peak_step / total, "unit": "% of MI355X peak",
        "ms_per_step": total * 1e3, "cores": len(os.sched_getaffinity(0)), "kind": "oracle",
        "sample": "rmsnorm 1024/65536 rows x64; gemm 256/2048 rows x8; attention 4/64 sequences "
                  "scaled by context length; logsoftmax 16/64 rows x4 (numpy fp64 / fp32 tree replay)",
        "per_op_s": {k: round(v, 4) for k, v in est.items()},
    }


def measured_traffic(root):
    """HBM bytes per call of the dominant kernel from the committed rocprofv3 counter summary
    (profiles/attention_decode_traffic.json), or None if the kernel source changed since."""
    import hashlib
    try:
        rec = json.load(open(os.path.join(root, "profiles", "attention_decode_traffic.json")))
        src = open(os.path.join(root, rec["source"]), "rb").read()
    except (OSError, ValueError, KeyError):
        return None
    if hashlib.sha256(src).hexdigest() != rec.get("source_sha256"):
        return None
    return int(rec["traffic_bytes"])


def gemm_profile(torch, bi, shape):
    """One Mistral-shaped bi_gemm (A [M, K], W [N, K] bf16 ~N(0,1)), timed with HIP events."""
    M, N, K = shape
    g = torch.Generator(device="cuda:0").manual_seed(7)
    A = torch.randn((M, K), generator=g, device="cuda:0").to(torch.bfloat16)
    W = torch.randn((N, K), generator=g, device="cuda:0").to(torch.bfloat16)
    C = torch.empty((M, N), dtype=torch.bfloat16, device="cuda:0")
    for _ in range(5):
        bi.bi_gemm(A, W, out=C)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(20):
        bi.bi_gemm(A, W, out=C)
    e1.record()
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) / 20 * 1e-3
    print(json.dumps({"gemm": [M, N, K], "tile": list(bi.bi_gemm_tile(M, N, K)),
                      "ms": round(t * 1e3, 4), "TFLOPs": round(2 * M * N * K / t / 1e12, 1)}), flush=True)


def gemm_sweep(torch, bi):
    """Mistral-shaped GEMMs (N, K) x M, TFLOP/s of bi_gemm and of the split-K variant."""
    dev = "cuda:0"
    out = []
    for (N, K) in [(6144, 4096), (4096, 4096), (28672, 4096), (4096, 14336), (32000, 4096)]:
        W = torch.randn((N, K), device=dev).to(torch.bfloat16)
        for M in (1, 64, 1024, 2048, 4096, 8192, 16384):
            A = torch.randn((M, K), device=dev).to(torch.bfloat16)
            C = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
            res = {}
            for name, fn in (("bi_gemm", lambda: bi.bi_gemm(A, W, out=C)),
                             ("splitk", lambda: bi.bi_gemm_splitk(A, W, out=C))):
                for _ in range(3):
                    fn()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                reps = 20
                e0.record()
                for _ in range(reps):
                    fn()
                e1.record(); torch.cuda.synchronize()
                t = e0.elapsed_time(e1) / reps * 1e-3
                res[name] = dict(ms=t * 1e3, tflops=2.0 * M * N * K / t / 1e12)
            out.append(dict(N=N, K=K, M=M, **{k: {kk: round(vv, 4) for kk, vv in v.items()} for k, v in res.items()},
                            frac_of_peak=round(res["bi_gemm"]["tflops"] * 1e12 / BF16_PEAK, 4)))
            print(json.dumps(out[-1]), flush=True)
            del A, C
        del W
    return out


def model_bench(torch, bi):
    """The composition rows: 32-layer Mistral-7B-shaped greedy decoding (random bf16 weights,
    std 0.02) of a 1400-token prompt alone and inside a ragged batch of 49 prompts, as in the
    batch-invariance test.  Prefill time = a 1-token generation; decode step = the difference
    between a 17- and a 1-token generation over 16 steps.  Reported, not graded."""
    import synth
    from invariant_amd.model import Dims, PagedKVCache, greedy_generate, random_model
    dims = Dims()
    model = random_model(dims, seed=5)
    prompt = synth.uniform_ints(1400, 0, 31999, 5, 0)
    lens = synth.ragged_lengths(48, 200, 4000, 5, 1)
    others = [synth.uniform_ints(int(L), 0, 31999, 5, 10 + i) for i, L in enumerate(lens)]
    prompts = others[:24] + [prompt] + others[24:]
    total = sum(len(p) + 64 for p in prompts)
    cache = PagedKVCache(dims, n_pages=total // 16 + 2 * len(prompts) + 16, seed=5)

    def timed(ps, n):
        torch.cuda.synchronize()
        t = time.perf_counter()
        greedy_generate(model, ps, n, cache, dims)
        torch.cuda.synchronize()
        return time.perf_counter() - t

    timed([prompt], 2)
    # bytes a decode step reads: every weight except the gate-then-up copy of the MLP rows
    # (decoding reads their interleaved copy)
    weight_bytes = sum(t.numel() * t.element_size() for t in _tensors(model)) - sum(
        w["wgate_up"].numel() * 2 for w in model["layers"])
    out_layer = layer_bench(torch, model, dims)
    out = {"workload": "Mistral-7B-shaped 32-layer greedy decode, random bf16 weights",
           "weight_bytes": weight_bytes, "decoder_layer_decode": out_layer}
    for name, ps in (("alone_1x1400", [prompt]), ("batched_49_ragged", prompts)):
        t1 = timed(ps, 1)
        t17 = timed(ps, 17)
        step = (t17 - t1) / 16
        ntok = sum(len(p) for p in ps)
        out[name] = dict(prefill_tokens=ntok, prefill_s=round(t1, 4),
                         prefill_tokens_per_s=round(ntok / t1, 1),
                         decode_step_ms=round(step * 1e3, 3),
                         decode_tokens_per_s=round(len(ps) / step, 1),
                         decode_weight_GBps=round(weight_bytes / step / 1e9, 1))
        log(name, out[name])
    print(json.dumps(out), flush=True)


def layer_bench(torch, model, dims):
    """One decoder layer at decode: B requests with contexts L ~ U[0, 4096] (cache pages
    reserved, contents as they are), one new token each; time per layer call."""
    import synth
    from invariant_amd.model import PagedKVCache, decoder_layer, make_batch
    out = {}
    layer = model["layers"][0]
    ctx = synth.ragged_lengths(256, 0, 4096, 3, 2)
    cache = PagedKVCache(dims, n_pages=int(ctx.sum()) // 16 + 2 * 256 + 16, seed=3, n_layers=1)
    lw_bytes = sum(t.numel() * t.element_size() for t in _tensors(layer)) - layer["wgate_up"].numel() * 2
    for B in (1, 8, 64, 256):
        sids = list(range(B))
        batch = make_batch(cache, sids, [int(c) for c in ctx[:B]],
                           [np.asarray([7], np.int32)] * B, dims=dims)
        h = torch.randn((B, dims.hidden), device="cuda").to(torch.bfloat16)
        f = lambda: decoder_layer(layer, h, batch, cache.k[0], cache.v[0], dims)
        for _ in range(3):
            f()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(20):
            f()
        e1.record()
        torch.cuda.synchronize()
        t = e0.elapsed_time(e1) / 20 * 1e-3
        kv = 2 * 2 * dims.n_kv_heads * dims.head_dim * int(ctx[:B].sum() + B)
        out[f"B{B}"] = dict(us=round(t * 1e6, 1), weight_GBps=round(lw_bytes / t / 1e9, 1),
                            weights_plus_kv_GBps=round((lw_bytes + kv) / t / 1e9, 1))
        log("layer", B, out[f"B{B}"])
        for sid in sids:
            cache.release(sid)
    return out


def _tensors(obj):
    import torch
    if isinstance(obj, torch.Tensor):
        yield obj
    elif isinstance(obj, dict):
        for v in obj.values():
            yield from _tensors(v)
    elif isinstance(obj, (list, tuple)):
        for v in obj:
            yield from _tensors(v)
    elif hasattr(obj, "__dict__"):
        for v in vars(obj).values():
            yield from _tensors(v)


def graph_step(torch, inp, ops, K):
    """The same step captured once as a HIP graph (its kernel launches replayed as one) and
    timed over K replays.  Every output of a replay must equal the eager step's bit for bit;
    otherwise (or if capture fails) the eager time stands."""
    names = ("y", "C", "attn_out", "lp", "am")
    eager = {k: inp[k].clone() for k in names}
    try:
        graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for _, fn in ops:
                fn()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        with torch.cuda.graph(graph):
            for _, fn in ops:
                fn()
        for k in names:
            inp[k].zero_()
        graph.replay()
        torch.cuda.synchronize()
    except Exception as e:  # noqa: BLE001 - report and keep the eager figure
        return None, f"eager (graph capture failed: {type(e).__name__})"
    if not all(torch.equal(inp[k].view(torch.uint8), eager[k].view(torch.uint8)) for k in names):
        return None, "eager (graph replay differed from the eager step)"
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(K):
        graph.replay()
    torch.cuda.synchronize()
    t = (time.perf_counter() - t0) / K
    ok = all(torch.equal(inp[k].view(torch.uint8), eager[k].view(torch.uint8)) for k in names)
    if not ok:
        return None, "eager (graph replay differed from the eager step)"
    return t, "hip graph of the step's kernels, every replay's outputs equal to the eager step's"


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--gemm-sweep", action="store_true")
    ap.add_argument("--gemm-profile", metavar="M,N,K",
                    help="run bi_gemm on one shape (5 warm-up + 20 timed calls) and print its "
                         "TFLOP/s, for rocprofv3 counter runs")
    ap.add_argument("--model", action="store_true",
                    help="time 32-layer greedy decoding alone and in a 49-prompt batch (reported)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (to scale rocprof byte counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this path has no collectives and every box has "
              "one MI355X; run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU (MI355X)")
    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    import invariant_amd as bi
    bi.load()

    if args.gemm_sweep:
        gemm_sweep(torch, bi)
        return
    if args.model:
        model_bench(torch, bi)
        return
    if args.gemm_profile:
        gemm_profile(torch, bi, [int(v) for v in args.gemm_profile.split(",")])
        return

    if args.copy_calibration:
        src = torch.ones((1 << 29,), dtype=torch.bfloat16, device="cuda:0")   # 1 GiB
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    log("building inputs")
    inp = build_inputs(torch, bi)
    ops = step_ops(bi, inp)
    wk = work(inp)
    for _ in range(args.warmup):
        for _, fn in ops:
            fn()
    torch.cuda.synchronize()

    K = args.steps
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in ops]
          for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(K):
        for j, (_, fn) in enumerate(ops):
            ev[s][j][0].record()
            fn()
            ev[s][j][1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = {name: float(np.mean([ev[s][j][0].elapsed_time(ev[s][j][1]) for s in range(K)])) * 1e-3
           for j, (name, _) in enumerate(ops)}
    eager_step_s = wall / K
    graph_step_s, graph_note = graph_step(torch, inp, ops, K)
    step_s = graph_step_s if graph_step_s is not None else eager_step_s

    comps = {}
    t_peak = 0.0
    for name, w in wk.items():
        tp = w["flops"] / BF16_PEAK if w["bound"] == "mfma" else w["bytes"] / HBM_PEAK
        t_peak += tp
        comps[name] = dict(ms=round(per[name] * 1e3, 5), GBps=round(w["bytes"] / per[name] / 1e9, 2),
                           TFLOPs=round(w["flops"] / per[name] / 1e12, 2), bound=w["bound"],
                           frac=round(tp / per[name], 4))
    kernel_sum = sum(per.values())
    att = wk["attention_decode"]
    res = {
        "metric": METRIC,
        "value": round(100.0 * t_peak / step_s, 3),
        "unit": "% of MI355X peak",
        "n_gpus": 1, "steps": K, "warmup": args.warmup,
        "ms_per_step": round(step_s * 1e3, 4),
        "eager_ms_per_step": round(eager_step_s * 1e3, 4),
        "step_launch": graph_note,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "hot-path pass: bi_rmsnorm x[65536,4096] + bi_gemm 2048^3 + "
                               "bi_attention decode B=64 ctx~U[1400,32768] GQA 32/8 d128 page16 + "
                               "bi_logsoftmax_argmax [64,32000]",
                   "global_batch": 64, "seq_len": int(inp["L"].max()), "parallelism": "none (1 GPU)"},
        "components": comps,
        "roofline": {"kernel": "bi_attention decode (kv_write + attn_split + attn_combine)",
                     "bound": "hbm", "achieved": round(att["bytes"] / per["attention_decode"] / 1e9, 1),
                     "peak": HBM_PEAK / 1e9, "unit": "GB/s",
                     "frac": round(att["bytes"] / per["attention_decode"] / HBM_PEAK, 4),
                     "traffic": measured_traffic(os.path.dirname(os.path.abspath(__file__))),
                     "algorithmic_bytes": att["bytes"]},
        "kernel_time_ms": round(kernel_sum * 1e3, 4),
    }
    # non-invariant comparison variants on the same inputs (the cost of invariance)
    L = inp["L"]
    total_chunks = int(sum((int(l) - 1) // 256 + 1 for l in L))
    variants = [
        ("gemm", "bi_gemm_splitk", lambda: bi.bi_gemm_splitk(inp["A"], inp["B_nk"], out=inp["C"])),
        ("attention_decode", "bi_attention_batchdep_split", lambda: bi.bi_attention_batchdep_split(
            inp["q"], inp["k_new"], inp["v_new"], inp["k_cache"], inp["v_cache"], inp["bt"],
            inp["seq_lens"], inp["qsl"], int(L.max()), total_chunks, 1.0 / np.sqrt(128.0),
            out=inp["attn_out"], workspace=inp["ws"])),
    ]
    comp = {}
    for name, vname, fn in variants:
        for _ in range(2):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(K):
            fn()
        e1.record()
        torch.cuda.synchronize()
        t = e0.elapsed_time(e1) / K * 1e-3
        comp[name] = dict(variant=vname, ms=round(t * 1e3, 5),
                          invariant_ms=round(per[name] * 1e3, 5),
                          invariant_slowdown=round(per[name] / t, 4))
    res["nonbi_comparison"] = comp
    if not args.no_cpu_baseline:
        log("timing the oracle on a sample")
        res["cpu_baseline"] = cpu_baseline(inp, torch, wk, t_peak)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
