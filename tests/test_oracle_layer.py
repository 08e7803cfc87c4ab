"""Pins of the decoder-layer oracle pieces (CPU only, small dimensions).

Cited: "Defeating nondeterminism in LLM inference", section on making kernels
batch-invariant (pointwise operations around the three reductions); readings for RoPE
(rotate-half pairing, base 10000) and SwiGLU are stated in oracle/layer.py.
"""
import math

import numpy as np

from oracle import fp
from oracle.layer import decoder_layer_ref, rope_angles, rope_f64, swiglu_f64


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
    x = fp.bf16_to_f64(inter["x"])
    assert np.array_equal(inter["attn"].reshape(1, d), x)
    assert np.array_equal(out, fp.bf16_to_f64(fp.f64_to_bf16(fp.bf16_to_f64(h) + x)))
