"""Host-side checks of the C-ABI library (no GPU needed, no kernel launched).

The library must load, export every entry point include/bi.h declares, report its
compile-time strategy, and reject invalid arguments before touching the GPU (the page
on verifying GPU programs: validation data with wrong shapes and illegal types).
"""
import ctypes
import os
import re

import numpy as np
import pytest

import invariant_amd as bi
from oracle.logsoftmax import K as ORACLE_K

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "bi.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(bi_[a-z_0-9]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(bi.LIB_PATH):
        import invariant_amd.build as b
        b.build()
    return bi.load()


def test_every_declared_symbol_is_exported(lib):
    names = _declared()
    assert len(names) >= 13
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(bi.EXPORTS)


def test_config_and_status_strings(lib):
    cfg = bi.get_config()
    assert cfg["tree_max_lanes"] == 256 and cfg["wave_size"] == 64 and cfg["attn_chunk"] == 256
    assert (cfg["gemm_mfma_m"], cfg["gemm_mfma_n"], cfg["gemm_mfma_k"]) == (16, 16, 32)
    assert cfg["version"] == 3 and cfg["attn_merge_group"] == 4 and cfg["gemm_tile_k"] == 64
    assert bi.status_string(0) == "BI_OK" and bi.status_string(-2) == "BI_ERR_SHAPE"
    assert bi.status_string(-99) == "BI_ERR_UNKNOWN"
    assert lib.bi_get_config(None) == -1


def test_validation_rejects_before_launch(lib):
    P = ctypes.c_void_p(16)           # never dereferenced: validation fails first
    assert lib.bi_rmsnorm(P, P, P, 4, 8, 8, 8, 1e-6, 7, 1, None) == -3
    assert lib.bi_rmsnorm(P, P, P, -1, 8, 8, 8, 1e-6, 1, 1, None) == -2
    assert lib.bi_rmsnorm(P, P, P, 4, 8, 4, 8, 1e-6, 1, 1, None) == -2
    assert lib.bi_rmsnorm(None, P, P, 4, 8, 8, 8, 1e-6, 1, 1, None) == -1
    assert lib.bi_rmsnorm(None, None, None, 0, 8, 8, 8, 1e-6, 1, 1, None) == 0
    assert lib.bi_gemm(P, P, P, 4, 4, 8, 8, 8, 4, 5, 1, 1, None) == -3
    assert lib.bi_gemm(P, P, P, 4, 4, 0, 8, 8, 4, 1, 1, 1, None) == -2
    assert lib.bi_gemm(ctypes.c_void_p(18), P, P, 4, 4, 8, 8, 8, 4, 1, 1, 1, None) == -4
    assert lib.bi_gemm(P, P, P, 4, 4, 8, 9, 8, 4, 1, 1, 1, None) == -4
    assert lib.bi_gemm(None, P, P, 4, 4, 8, 8, 8, 4, 1, 1, 1, None) == -1
    # fused gate/up + SwiGLU: F must be a multiple of 16; null and misaligned operands
    assert lib.bi_gemm_swiglu(P, P, P, 4, 24, 64, 64, 64, 24, None) == -2
    assert lib.bi_gemm_swiglu(P, P, P, 4, 32, 64, 60, 64, 32, None) == -2
    assert lib.bi_gemm_swiglu(None, P, P, 4, 32, 64, 64, 64, 32, None) == -1
    assert lib.bi_gemm_swiglu(P, ctypes.c_void_p(18), P, 4, 32, 64, 64, 64, 32, None) == -4
    assert lib.bi_gemm_swiglu(None, None, None, 0, 32, 64, 64, 64, 32, None) == 0
    # fused residual add + RMSNorm: dtype, D a multiple of 8 up to 8192, null operands
    assert lib.bi_add_rmsnorm(P, P, P, 3, P, P, 1, 4, 64, 1e-5, None) == -3
    assert lib.bi_add_rmsnorm(P, P, P, 1, P, P, 1, 4, 60, 1e-5, None) == -6
    assert lib.bi_add_rmsnorm(P, P, P, 1, P, P, 1, 4, 8200, 1e-5, None) == -6
    assert lib.bi_add_rmsnorm(P, None, P, 1, P, P, 1, 4, 64, 1e-5, None) == -1
    assert lib.bi_add_rmsnorm(P, P, P, 1, P, P, 1, -1, 64, 1e-5, None) == -2
    assert lib.bi_logsoftmax_argmax(P, 2, 10, 8, None, P, None) == -2
    assert lib.bi_logsoftmax_argmax(None, 2, 10, 12, None, P, None) == -1
    assert lib.bi_logsoftmax_argmax(P, 2, 1024, 1024, P, P, None) == -2   # logprobs over logits
    # attention: unsupported head_dim, group, page size; missing workspace
    args = [P] * 8
    def att(T=4, hq=32, hkv=8, d=128, ps=16, maxp=4, msl=64, ws=None, wsz=0, B=2):
        return lib.bi_attention(*args, B, T, hq, hkv, d, ps, maxp, msl, 0.088, P, 1, ws, wsz, None)
    assert att(d=64) == -6
    assert att(hq=24, hkv=8) == -6
    assert att(hq=30, hkv=8) == -2
    assert att(ps=24) == -6
    assert att(msl=65) == -2
    assert att() == -5
    assert lib.bi_attention_workspace_bytes(4, 32, 128, 64) == (4 * 32 * 1 * 2 + 4 * 32 * 128) * 4 + 4 * 16
    assert lib.bi_attention_workspace_bytes(2000, 32, 128, 64) == 0
    assert lib.bi_gemm_splitk_workspace_bytes(2048, 2048, 2048) == 2 * 2048 * 2048 * 4


def test_hip_constants_equal_oracle_derivation():
    """The EXP/LOG constants written as bit patterns in the HIP source are the values the
    oracle derives from exact rationals (the two sides share no code)."""
    src = open(os.path.join(ROOT, "invariant_amd", "csrc", "logsoftmax.hip")).read()
    hexes = set(int(h, 16) for h in re.findall(r"f32c\((0x[0-9a-f]+)u\)", src))
    want = [ORACLE_K["LOG2E"], ORACLE_K["LN2_HI"], ORACLE_K["LN2_LO"], ORACLE_K["SQRT2"],
            *ORACLE_K["EXP_C"], *ORACLE_K["LOG_B"]]
    for w in want:
        assert int(np.float32(w).view(np.uint32)) in hexes, w
