"""Exhaustive device sweeps of the fp32 functions whose bits are part of the contract, each
against the oracle's replay on every float of its domain ("How to verify GPU program
correctness before deployment", sections on preparing validation data and testing many
scenarios: every value of the domain rather than those a row test happens to produce):

  EXP over every float in [-104, 0] (and +0)      vs the oracle's Cody-Waite replay
  LOG over every float in [1, 32768]              vs the oracle's atanh-series replay
  sqrt, 1/x and x/14336 over every positive float vs numpy binary32 (correctly rounded),
                                                    the operations of RMSNorm's scale
  RMSNorm's scale r = 1/sqrt(ssum/D + eps)        on 16M random (ssum, D) pairs

The device side is a test-only library (tests/hip/libfpsweep.so) built from the same
header the kernels include; the oracle side is oracle/explog.c, pinned to the Python oracle
in tests/test_oracle_logsoftmax.py.
"""
import ctypes
import os

import numpy as np
import pytest
import torch

from oracle import explog_c
from tests._gpu import say

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))
CHUNK = 1 << 26


@pytest.fixture(scope="module")
def fps():
    path = os.path.join(HERE, "hip", "libfpsweep.so")
    if not os.path.exists(path):
        raise RuntimeError("tests/hip/libfpsweep.so is not built: run __graft_entry__.build()")
    lib = ctypes.CDLL(path)
    lib.fps_sweep.argtypes = [ctypes.c_uint32, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.fps_rms_scale.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_float, ctypes.c_int64,
                                  ctypes.c_void_p, ctypes.c_void_p]
    return lib


def _sweep(fps, fn, first, last, oracle):
    """Every float with bits first..last (inclusive) through device function fn, chunk by
    chunk, bitwise against oracle(first_bits, n) -> float32 array."""
    buf = torch.empty(CHUNK, dtype=torch.float32, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    total, bad = 0, 0
    b = first
    while b <= last:
        n = min(CHUNK, last - b + 1)
        assert fps.fps_sweep(ctypes.c_uint32(b), n, fn, ctypes.c_void_p(buf.data_ptr()), stream) == 0
        got = buf[:n].cpu().numpy().view(np.uint32)
        want = oracle(b, n).view(np.uint32)
        diff = np.flatnonzero(got != want)
        if diff.size:
            i = int(diff[0])
            say("mismatch at bits", hex(b + i), "got", hex(int(got[i])), "want", hex(int(want[i])))
            bad += int(diff.size)
        total += n
        b += n
    return total, bad


def _np_unary(f):
    def run(first, n):
        x = (np.arange(n, dtype=np.uint64) + np.uint64(first)).astype(np.uint32).view(np.float32)
        with np.errstate(all="ignore"):
            return f(x).astype(np.float32)
    return run


def test_exp_every_float_in_domain(fps):
    n, bad = _sweep(fps, 0, 0x80000000, 0xC2D00000, explog_c.exp_bits)    # -0 .. -104
    n0, bad0 = _sweep(fps, 0, 0x00000000, 0x00000000, explog_c.exp_bits)  # +0
    say("EXP", n + n0, "floats, mismatches", bad + bad0)
    assert bad == 0 and bad0 == 0 and n == 0x42D00001


def test_log_every_float_in_domain(fps):
    n, bad = _sweep(fps, 1, 0x3F800000, 0x47000000, explog_c.log_bits)     # 1 .. 32768
    say("LOG", n, "floats, mismatches", bad)
    assert bad == 0 and n == 0x07800001


@pytest.mark.parametrize("fn,name,f", [(2, "sqrt", np.sqrt), (3, "1/x", lambda x: np.float32(1.0) / x),
                                       (4, "x/14336", lambda x: x / np.float32(14336.0))])
def test_rmsnorm_operations_every_positive_float(fps, fn, name, f):
    # every positive float, denormals included, and the infinity
    n, bad = _sweep(fps, fn, 0x00000000, 0x7F800000, _np_unary(f))
    say(name, n, "floats, mismatches", bad)
    assert bad == 0


def test_rms_scale_random(fps):
    rng = np.random.default_rng(70)
    m = 1 << 24
    d = rng.choice(np.asarray([512, 4096, 14336, 1000, 9000], dtype=np.int32), m)
    ssum = (rng.random(m) * np.asarray([1e-3, 1.0, 1e4, 1e8])[rng.integers(0, 4, m)] * d).astype(np.float32)
    out = torch.empty(m, dtype=torch.float32, device="cuda")
    S, D = torch.from_numpy(ssum).cuda(), torch.from_numpy(d).cuda()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    for eps in (1e-5, 1e-6):
        assert fps.fps_rms_scale(ctypes.c_void_p(S.data_ptr()), ctypes.c_void_p(D.data_ptr()), eps, m,
                                 ctypes.c_void_p(out.data_ptr()), stream) == 0
        mean = ssum / d.astype(np.float32)
        want = np.float32(1.0) / np.sqrt(mean + np.float32(eps))
        assert np.array_equal(out.cpu().numpy().view(np.uint32), want.view(np.uint32)), eps
