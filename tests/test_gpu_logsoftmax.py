"""bi_logsoftmax_argmax on the GPU: logprobs and argmax bit-exact against the oracle.

Cited: greedy decoding and token probabilities ("Does the same LLM give different
outputs on different GPUs? Why?"); near-tie argmax ("Same model, same input, different
answer").
"""
import numpy as np
import pytest
import torch

from oracle.logsoftmax import logsoftmax_argmax
from tests._gpu import f32, host, same_bits, say

pytestmark = pytest.mark.gpu


def _cmp(lib, x):
    lp, am = lib.bi_logsoftmax_argmax(f32(x))
    rlp, ram = logsoftmax_argmax(x)
    assert np.array_equal(host(am), ram)
    got = host(lp)
    nan = np.isnan(rlp)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), rlp[~nan].view(np.uint32))


@pytest.mark.parametrize("m,v", [(1, 32000), (49, 32000), (3, 1000), (2, 37), (5, 4099), (1, 1), (2, 262144),
                                 (4, 32768), (3, 1024), (2, 1020), (2, 8196), (2, 32772)])
def test_bit_exact(lib, m, v):
    say("logsoftmax", m, v)
    rng = np.random.default_rng(m * 7 + v)
    x = (rng.standard_normal((m, v)) * 1.3).astype(np.float32)
    _cmp(lib, x)


def test_special_rows(lib):
    v = 32000
    x = np.zeros((7, v), dtype=np.float32)
    x[0, 5] = x[0, 9] = 2.0                          # tie -> 5
    x[1, 3] = np.float32(3.4819); x[1, 31000] = np.float32(3.4821)
    x[2, 6] = np.nan; x[2, 2] = np.nan
    x[3, :] = -0.0; x[3, 4] = 0.0
    x[4, :] = -np.inf; x[4, 100] = 1.0
    x[5, 17] = 150.0
    x[6] = np.random.default_rng(0).standard_normal(v).astype(np.float32) * 40
    # rows whose candidates lie in different parts of the row (the split form reduces the
    # maximum across workgroups): far ties, a late NaN after an early maximum, all NaN,
    # +inf, the maximum in the last element
    y = (np.random.default_rng(1).standard_normal((6, v)) * 2).astype(np.float32)
    y[0, 300] = y[0, 31999] = y[0, 17000] = 9.0      # tie -> 300
    y[1, 2] = 50.0; y[1, 29999] = np.nan             # NaN wins -> 29999
    y[2, :] = np.nan
    y[3, 8000] = np.inf; y[3, 8001] = np.inf         # -> 8000, logprobs NaN / -inf
    y[4, v - 1] = 30.0
    y[5, :] = -np.inf; y[5, 70] = -0.0; y[5, 4000] = 0.0   # -> 70
    x = np.concatenate([x, y])
    _cmp(lib, x)
    _, only = lib.bi_logsoftmax_argmax(f32(x), want_logprobs=False)
    assert np.array_equal(host(only), logsoftmax_argmax(x)[1])


def test_batch_invariance_and_repeats(lib):
    x = (np.random.default_rng(3).standard_normal((64, 32000)) * 2).astype(np.float32)
    X = f32(x)
    lp, am = lib.bi_logsoftmax_argmax(X)
    for m in (1, 2, 17, 49):
        lpm, amm = lib.bi_logsoftmax_argmax(X[:m].contiguous())
        assert same_bits(lpm, lp[:m]) and torch.equal(amm, am[:m])
    for _ in range(50):
        l2, a2 = lib.bi_logsoftmax_argmax(X)
        assert same_bits(l2, lp) and torch.equal(a2, am)
    _, only = lib.bi_logsoftmax_argmax(X, want_logprobs=False)
    assert torch.equal(only, am)


def test_row_stride(lib):
    # rows ld = V + 4 apart (a view of a wider buffer): logprobs come back with the same stride
    for v in (32000, 4099):
        x = (np.random.default_rng(v).standard_normal((5, v + 4)) * 1.7).astype(np.float32)
        X = f32(x)[:, :v]
        lp, am = lib.bi_logsoftmax_argmax(X)
        assert lp.stride(0) == v + 4
        rlp, ram = logsoftmax_argmax(np.ascontiguousarray(x[:, :v]))
        assert np.array_equal(host(am), ram)
        assert np.array_equal(host(lp).view(np.uint32), rlp.view(np.uint32))
