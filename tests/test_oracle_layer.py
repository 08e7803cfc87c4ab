"""Pins of the decoder-layer and model oracle (CPU only, small dimensions).

Cited: "Defeating nondeterminism in LLM inference", section on making kernels
batch-invariant (pointwise operations around the three reductions) and on batch-invariant
attention (a token reduces over the same keys in a prefill and in a decode); the arXiv
abstract on cross-vendor mismatch (upcasting to FP32 except the MLPs lowers the error);
readings for RoPE (rotate-half pairing, base 10000) and SwiGLU are stated in
oracle/layer.py.
"""
import math

import numpy as np

from oracle import fp
from oracle.layer import (Spec, decoder_layer_ref, head_ref, model_ref_forward, model_ref_logits,
                          rope_angles, rope_f64, sequence_layer_ref, swiglu_f64)


def test_rope_is_complex_rotation():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((3, 2, 16))
    pos = [0, 5, 1000]
    y = rope_f64(x, pos, 10000.0)
    for t, p in enumerate(pos):
        for i in range(8):
            theta = p * 10000.0 ** (-2 * i / 16)
            z = complex(x[t, 0, i], x[t, 0, i + 8]) * complex(math.cos(theta), math.sin(theta))
            assert abs(y[t, 0, i] - z.real) < 1e-12 and abs(y[t, 0, i + 8] - z.imag) < 1e-12
    assert np.allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1))
    assert np.array_equal(rope_f64(x, [0, 0, 0]), x)
    assert rope_angles([7], 16)[0, 0] == 7.0


def test_swiglu_special_values():
    g = np.array([0.0, 50.0, -50.0, 1.0])
    u = np.array([3.0, 2.0, 2.0, 1.0])
    s = swiglu_f64(g, u)
    assert s[0] == 0.0 and abs(s[1] - 100.0) < 1e-12 and abs(s[2]) < 1e-18
    assert abs(s[3] - 1.0 / (1.0 + math.exp(-1.0))) < 1e-15


def _small(seed, d=64, hq=4, hkv=2, hd=16, ffn=96):
    rng = np.random.default_rng(seed)
    b = lambda *shape, sd=0.1, mean=0.0: fp.f32_to_bf16((rng.standard_normal(shape) * sd + mean).astype(np.float32))
    w = dict(attn_norm=b(d, sd=0.02, mean=1.0), wqkv=b((hq + 2 * hkv) * hd, d), wo=b(d, hq * hd),
             ffn_norm=b(d, sd=0.02, mean=1.0), wgate_up=b(2 * ffn, d), wdown=b(d, ffn))
    return w, b


def test_zero_output_projections_leave_the_residual():
    w, b = _small(1)
    w["wo"][:] = 0
    w["wdown"][:] = 0
    h = b(3, 64, sd=1.0)
    pk = [b(p, 2, 16, sd=1.0) for p in (0, 4, 9)]
    pv = [b(p, 2, 16, sd=1.0) for p in (0, 4, 9)]
    out, _ = decoder_layer_ref(h, w, [0, 4, 9], pk, pv, 1e-5, 10000.0, 4, 2, 16)
    assert np.array_equal(out, fp.bf16_to_f64(h))


def test_first_token_attention_is_its_value():
    # one token at position 0 attends only to itself: the attention output is v, and
    # with V projection = identity rows and Wo = identity, h2 = h + x_normed (rounded)
    d, hq, hkv, hd = 64, 4, 4, 16
    w, b = _small(2, d, hq, hkv, hd)
    wqkv = fp.bf16_to_f64(w["wqkv"]).copy()
    wqkv[2 * d:, :] = np.eye(d)                       # v = x
    w["wqkv"] = fp.f64_to_bf16(wqkv)
    w["wo"] = fp.f64_to_bf16(np.eye(d))
    w["wdown"][:] = 0
    h = b(1, d, sd=1.0)
    out, inter = decoder_layer_ref(h, w, [0], [np.zeros((0, hkv, hd), np.uint16)],
                                   [np.zeros((0, hkv, hd), np.uint16)], 1e-5, 10000.0, hq, hkv, hd)
    x = inter["x"]
    assert np.array_equal(inter["attn"].reshape(1, d), x)
    assert np.array_equal(out, fp.bf16_to_f64(fp.f64_to_bf16(fp.bf16_to_f64(h) + x)))


DIMS = dict(n_q_heads=4, n_kv_heads=2, head_dim=16)


def _small_model(seed, n_layers=2, d=64, ffn=96, vocab=50):
    rng = np.random.default_rng(seed)
    b = lambda *shape, sd=0.1, mean=0.0: fp.f32_to_bf16((rng.standard_normal(shape) * sd + mean).astype(np.float32))
    layers = []
    for _ in range(n_layers):
        w, _ = _small(int(rng.integers(1 << 30)), d, 4, 2, 16, ffn)
        layers.append(w)
    return dict(embed=b(vocab, d, sd=1.0), layers=layers, final_norm=b(d, sd=0.02, mean=1.0),
                lm_head=b(vocab, d))


def test_sequence_form_equals_independent_token_form():
    # token p of a sequence, run as an independent request whose prior context holds the
    # sequence's keys/values 0..p-1, gives the sequence form's row p
    w, b = _small(3)
    spec = Spec(**DIMS)
    h = fp.bf16_to_f64(b(9, 64, sd=1.0))
    out, inter = sequence_layer_ref(h, w, 0, np.zeros((0, 2, 16)), np.zeros((0, 2, 16)), spec)
    kb, vb = fp.f64_to_bf16(inter["k"]), fp.f64_to_bf16(inter["v"])
    for p in (0, 4, 8):
        o1, i1 = decoder_layer_ref(fp.f64_to_bf16(h[p:p + 1]), w, [p], [kb[:p]], [vb[:p]], 1e-5,
                                   10000.0, 4, 2, 16)
        assert np.allclose(o1[0], out[p], rtol=1e-12, atol=0), p
        assert np.allclose(i1["attn"][0], inter["attn"][p], rtol=1e-12, atol=1e-300), p


def test_one_layer_model_equals_layer_then_head():
    # the model oracle with one layer, teacher-forced, equals the independent-token layer
    # form (each step's prior context from the earlier steps) followed by the final norm
    # and the LM head, written out here step by step
    model = _small_model(4, n_layers=1)
    toks = [3, 17, 41, 0, 8]
    spec = Spec(**DIMS)
    got = model_ref_logits(toks[:3], toks[3:], model, **DIMS)
    ks = np.zeros((0, 2, 16), np.uint16)
    vs = np.zeros((0, 2, 16), np.uint16)
    rows = []
    for p, t in enumerate(toks):
        o, it = decoder_layer_ref(model["embed"][[t]], model["layers"][0], [p], [ks], [vs], 1e-5,
                                  10000.0, 4, 2, 16)
        ks = np.concatenate([ks, fp.f64_to_bf16(it["k"])])
        vs = np.concatenate([vs, fp.f64_to_bf16(it["v"])])
        if p >= 2:
            rows.append(head_ref(model, o, spec)[0])
    assert np.allclose(got, np.stack(rows), rtol=1e-12, atol=1e-12)


def test_teacher_forced_equals_one_pass_and_any_chunking():
    # the KV context grows piece by piece: decode steps, chunked prefill and one pass give
    # the same logits (a wrong position, a key appended twice or a missing cache row fails)
    model = _small_model(5)
    prompt = [1, 5, 9, 2, 33, 47, 12, 8, 30]
    forced = [4, 4, 19, 0]
    for variant in (False, True):
        a = model_ref_logits(prompt, forced, model, fp32_variant=variant, **DIMS)
        b = model_ref_logits(prompt, forced, model, fp32_variant=variant, one_pass=True, **DIMS)
        assert a.shape == (5, 50)
        assert np.allclose(a, b, rtol=1e-11, atol=1e-11), variant
        spec = Spec(**DIMS, variant=variant)
        seq = prompt + forced
        c = model_ref_forward([seq[:2], seq[2:7], seq[7:8], seq[8:]], model, spec,
                              logit_rows=lambda i, t: range(t))
        allrows = np.concatenate(c)
        assert np.allclose(allrows[len(prompt) - 1:], a, rtol=1e-11, atol=1e-11), variant
    # order matters (positions are applied): swapping two prompt tokens changes the logits
    sw = list(prompt)
    sw[0], sw[1] = sw[1], sw[0]
    assert not np.allclose(model_ref_logits(sw, [], model, **DIMS), a[:1])


def test_fp32_variant_storage_points():
    # zero output projections: the residual stream is the embedding, exactly, in both
    # models; the variant's logits are then fp32 norm -> fp32 x bf16 head in fp64, the bf16
    # model's come from a bf16-rounded norm output
    model = _small_model(6, n_layers=2)
    for w in model["layers"]:
        w["wo"][:] = 0
        w["wdown"][:] = 0
    toks = [7, 11, 13]
    e = fp.bf16_to_f64(model["embed"][toks])
    g = fp.bf16_to_f64(model["final_norm"])
    W = fp.bf16_to_f64(model["lm_head"])
    r = 1.0 / np.sqrt(np.mean(e * e, axis=1, keepdims=True) + 1e-5)
    exact = (e * r * g) @ W.T                       # fp64 definition of norm + head
    lv = model_ref_logits(toks, [], model, fp32_variant=True, one_pass=True, **DIMS)
    lb = model_ref_logits(toks, [], model, fp32_variant=False, one_pass=True, **DIMS)
    ev = np.abs(lv[-1] - exact[-1]).max()
    eb = np.abs(lb[-1] - exact[-1]).max()
    scale = np.abs(exact[-1]).max()
    assert ev < 1e-5 * scale                         # fp32 storage of the norm output
    assert eb > 1e-4 * scale and eb < 2e-2 * scale   # bf16 storage of the norm output


def _no_rounding_logits(model, toks):
    import oracle.layer as L
    saved = L.store
    try:
        L.store = lambda x, dtype: np.asarray(x, dtype=np.float64)
        return model_ref_logits(toks, [], model, one_pass=True, **DIMS)
    finally:
        L.store = saved


def test_fp32_variant_is_closer_to_fp64():
    # the cross-vendor abstract's claim, on this oracle: keeping the activations outside the
    # MLPs in fp32 moves the logits closer to a model with no storage rounding at all (with
    # and without the MLPs' contribution; the bf16 K/V cache bounds the gain)
    toks = [3, 1, 4, 1, 5, 9, 2, 6]
    for zero_mlp in (False, True):
        model = _small_model(7, n_layers=2)
        if zero_mlp:
            for w in model["layers"]:
                w["wdown"][:] = 0
        ref = _no_rounding_logits(model, toks)
        lv = model_ref_logits(toks, [], model, fp32_variant=True, one_pass=True, **DIMS)
        lb = model_ref_logits(toks, [], model, fp32_variant=False, one_pass=True, **DIMS)
        assert np.abs(lv - ref).mean() < np.abs(lb - ref).mean(), zero_mlp


def _is_bf16(x):
    return np.array_equal(fp.bf16_to_f64(fp.f64_to_bf16(x)), x)


def _is_f32(x):
    return np.array_equal(np.asarray(x, np.float32).astype(np.float64), x)


def test_storage_points_of_both_models():
    # which intermediates are stored in which type: bf16 model -- all bf16; variant --
    # x, qkv, q, attention output, o, h2 and the layer output fp32 (and not all bf16), k/v
    # (the cache) and the MLP (x2, gate/up, SwiGLU, down) bf16
    w, b = _small(8)
    h = fp.bf16_to_f64(b(6, 64, sd=1.0))
    z = np.zeros((0, 2, 16))
    out, it = sequence_layer_ref(h, w, 0, z, z, Spec(**DIMS))
    for name in ("x", "qkv", "q", "k", "v", "attn", "o", "h2", "x2", "gu", "mlp", "dn"):
        assert _is_bf16(it[name]), name
    assert _is_bf16(out)
    out, it = sequence_layer_ref(h, w, 0, z, z, Spec(**DIMS, variant=True))
    for name in ("x", "qkv", "attn", "o", "h2"):
        assert _is_f32(it[name]) and not _is_bf16(it[name]), name
    assert _is_f32(out) and not _is_bf16(out)
    assert _is_f32(it["q"]) and not _is_bf16(it["q"])
    for name in ("k", "v", "x2", "gu", "mlp", "dn"):
        assert _is_bf16(it[name]), name
    _, it = sequence_layer_ref(h, w, 0, z, z, Spec(**DIMS, variant=True, q_dtype="bf16"))
    assert _is_bf16(it["q"]) and _is_bf16(it["k"])
