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
    assert lib.bi_gemm_swiglu(P, P, P, 4, 24, 64, 64, 64, 24, 1, None) == -2
    assert lib.bi_gemm_swiglu(P, P, P, 4, 32, 64, 60, 64, 32, 1, None) == -2
    assert lib.bi_gemm_swiglu(None, P, P, 4, 32, 64, 64, 64, 32, 1, None) == -1
    assert lib.bi_gemm_swiglu(P, ctypes.c_void_p(18), P, 4, 32, 64, 64, 64, 32, 1, None) == -4
    assert lib.bi_gemm_swiglu(None, None, None, 0, 32, 64, 64, 64, 32, 1, None) == 0
    assert lib.bi_gemm_swiglu(P, P, P, 4, 32, 64, 64, 64, 32, 7, None) == -3     # w_layout
    # fused add + RMSNorm + projection: at most 4 rows, 1024 <= K <= 8192 (K % 8 == 0), the
    # sum apart from a and b; a, b, sum, gamma, W, C at distinct (never dereferenced) addresses
    a, b, sm, g, w, c = (ctypes.c_void_p(16 + (i << 24)) for i in range(6))
    ng = lib.bi_add_rmsnorm_gemm
    assert ng(a, b, sm, g, 1e-5, w, c, 1, 64, 1024, 1024, 64, 5, 1, None) == -3          # w_layout
    assert ng(a, b, sm, g, 1e-5, w, c, 1, 64, 1024, 1024, 64, 1, 7, None) == -3          # c_dtype
    assert ng(a, b, sm, g, 1e-5, w, c, 5, 64, 1024, 1024, 64, 1, 1, None) == -6          # 5 rows
    for k in (1028, 512, 8200):
        assert ng(a, b, sm, g, 1e-5, w, c, 1, 64, k, k, 64, 1, 1, None) == -6
    assert ng(a, b, sm, g, 1e-5, w, c, 3, 64, 8192, 8192, 64, 1, 1, None) == -6        # 48 KB of rows
    assert ng(a, b, sm, g, 1e-5, w, c, 1, 64, 1024, 1000, 64, 1, 1, None) == -2          # ldw < K
    assert ng(a, b, sm, g, 1e-5, w, c, 1, 64, 1024, 1024, 60, 1, 1, None) == -2          # ldc < N
    assert ng(None, b, sm, g, 1e-5, w, c, 1, 64, 1024, 1024, 64, 1, 1, None) == -1
    assert ng(a, ctypes.c_void_p(18), sm, g, 1e-5, w, c, 1, 64, 1024, 1024, 64, 1, 1, None) == -4
    assert ng(a, b, ctypes.c_void_p(16 + 1024), g, 1e-5, w, c, 1, 64, 1024, 1024, 64, 1, 1, None) == -2
    assert ng(a, b, b, g, 1e-5, w, c, 2, 64, 1024, 1024, 64, 2, 1, None) == -2          # sum is b
    assert ng(None, None, None, None, 1e-5, None, None, 0, 64, 1024, 1024, 64, 1, 1, None) == 0
    ns = lib.bi_add_rmsnorm_gemm_swiglu
    assert ns(a, b, sm, g, 1e-5, w, c, 1, 24, 1024, 1024, 24, 1, None) == -2             # F % 16
    assert ns(a, b, sm, g, 1e-5, w, c, 5, 32, 1024, 1024, 32, 2, None) == -6
    assert ns(a, b, sm, g, 1e-5, w, c, 1, 32, 1024, 1024, 32, 7, None) == -3
    assert ns(a, b, sm, g, 1e-5, None, c, 1, 32, 1024, 1024, 32, 1, None) == -1
    # tiled B / W: at most 64 rows, K a multiple of 8 and >= 1024, bf16 A
    assert lib.bi_gemm(P, P, P, 65, 64, 1024, 1024, 0, 64, 2, 1, 1, None) == -6
    assert lib.bi_gemm(P, P, P, 16, 64, 512, 512, 0, 64, 2, 1, 1, None) == -6
    assert lib.bi_gemm(P, P, P, 16, 64, 1028, 1032, 0, 64, 2, 1, 1, None) == -6
    assert lib.bi_gemm(P, P, P, 4, 64, 1024, 1024, 0, 64, 2, 2, 1, None) == -6    # fp32 A
    assert lib.bi_gemm(P, None, P, 4, 64, 1024, 1024, 0, 64, 2, 1, 1, None) == -1
    assert lib.bi_gemm_swiglu(P, P, P, 65, 32, 1024, 1024, 0, 32, 2, None) == -6
    assert lib.bi_pack_b_bytes(33, 1000) == 3 * 32 * 1024 and lib.bi_pack_b_bytes(0, 8) == 0
    # fixed split of K: k_slice a multiple of 64 and at least 64; the workspace holds one fp32
    # M x N partial per slice (none with one slice), checked before any launch
    fs, fsb = lib.bi_gemm_fixed_split, lib.bi_gemm_fixed_split_workspace_bytes
    assert fsb(3, 5, 4096, 1024) == 4 * 3 * 5 * 4 and fsb(3, 5, 4097, 1024) == 5 * 3 * 5 * 4
    assert fsb(3, 5, 1024, 1024) == 0 and fsb(3, 5, 4096, 100) == 0 and fsb(3, 5, 4096, 0) == 0
    for ks in (0, 32, 100, -64):
        assert fs(P, P, P, 4, 4, 4096, 4096, 4096, 4, 1, ks, P, 1 << 20, None) == -2
    assert fs(P, P, P, 4, 4, 4096, 4096, 4096, 4, 1, 1024, P, 255, None) == -5        # workspace
    assert fs(P, P, P, 4, 4, 4096, 4096, 4096, 4, 1, 1024, None, 1 << 20, None) == -5
    assert fs(P, P, P, 4, 4, 4096, 4096, 4096, 4, 9, 1024, P, 1 << 20, None) == -3    # c_dtype
    assert fs(None, P, P, 4, 4, 4096, 4096, 4096, 4, 1, 1024, P, 1 << 20, None) == -1
    assert fs(P, P, P, 4, 4, 4096, 4096, 4000, 4, 1, 1024, P, 1 << 20, None) == -2    # ldb < K
    assert fs(None, None, None, 0, 4, 4096, 4096, 4096, 4, 1, 1024, None, 0, None) == 0
    assert lib.bi_pack_b(P, 4, 64, 32, P, None) == -2
    assert lib.bi_pack_b(P, 4, 64, 64, ctypes.c_void_p(18), None) == -4
    assert lib.bi_pack_b(None, 4, 64, 64, P, None) == -1
    assert lib.bi_pack_b(None, 0, 64, 64, None, None) == 0
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
    args = [P, 1] + [P] * 7          # q (bf16), k_new, v_new, caches, table, lengths, offsets
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
    # the no-allocation form rejects a call whose partials exceed its 64 MiB scratch before
    # anything runs: 1024 tokens of 32768-token contexts need 1024*32*32*(2+128)*4 bytes
    assert lib.bi_attention_noalloc(*args, 1, 1024, 32, 8, 128, 16, 2048, 32768, 0.088, P, 1, None) == -5
    assert lib.bi_attention_noalloc(*args, 1, 4, 32, 8, 64, 16, 4, 64, 0.088, P, 1, None) == -6
    bad_q = [P, 7] + [P] * 7          # an unknown q dtype
    assert lib.bi_attention(*bad_q, 2, 4, 32, 8, 128, 16, 4, 64, 0.088, P, 1, P, 1 << 20, None) == -3
    assert lib.bi_rope_qkv(P, 6144, 1, P, P, 5, P, P, 4, 32, 8, 128, 10000.0, None) == -3
    # attention with exactly one of k_new, v_new NULL (both NULL means "in the cache already")
    one_null = [P, 1, None, P] + [P] * 5
    assert lib.bi_attention(*one_null, 2, 4, 32, 8, 128, 16, 4, 64, 0.088, P, 1, P, 1 << 20, None) == -1
    # fused RoPE + cache write: dtype, head_dim, page size, row stride, null operands
    def rkw(qd=1, ld=6144, d=128, ps=16, qkv=P, kc=P, T=4, B=2):
        return lib.bi_rope_kv_write(qkv, ld, 1, P, qd, kc, P, P, P, P, B, T, 32, 8, d, ps, 4, 10000.0, None)
    assert rkw(qd=5) == -3
    assert rkw(d=64, ld=3072) == -6
    assert rkw(ps=24) == -6
    assert rkw(ld=6000) == -2
    assert rkw(qkv=None) == -1
    assert rkw(kc=ctypes.c_void_p(18)) == -4
    assert rkw(T=0) == 0 and rkw(B=0) == 0
    # the comparison variant splits K only when the grid leaves CUs idle (256 CUs assumed
    # without a GPU): none for 2048^3 (256 tiles), four slices for 256 x 1024 (64 tiles)
    assert lib.bi_gemm_splitk_workspace_bytes(2048, 2048, 2048) == 0
    assert lib.bi_gemm_splitk_workspace_bytes(256, 1024, 8192) == 4 * 256 * 1024 * 4
    assert lib.bi_gemm_splitk_workspace_bytes(2, 1024, 2048) == 0      # split over 4 waves


def _fn_constants(src, name):
    """The f32c(0x...u) constants of device function `name`, in source order."""
    start = src.index(name + "(")
    body = src[src.index("{", start):]
    depth, end = 0, 0
    for i, ch in enumerate(body):
        depth += ch == "{"
        depth -= ch == "}"
        if depth == 0:
            end = i
            break
    return [int(h, 16) for h in re.findall(r"f32c\((0x[0-9a-f]+)u\)", body[:end])]


def _bits(v):
    return int(np.float32(v).view(np.uint32))


def test_hip_constants_equal_oracle_derivation():
    """The EXP/LOG constants written as bit patterns in the HIP source are the values the
    oracle derives from exact rationals (the two sides share no code), each in its role:
    EXP = 1/ln2, ln2 head, ln2 tail, then the Horner coefficients 1/7! .. 1/0!; LOG = sqrt 2,
    the Horner coefficients 2/15 .. 2/1, then ln2 head and tail.  A swap of two coefficients
    or of head and tail fails here."""
    src = open(os.path.join(ROOT, "invariant_amd", "csrc", "contract_fp.h")).read()
    k = ORACLE_K
    exp_want = [k["LOG2E"], k["LN2_HI"], k["LN2_LO"], *reversed(k["EXP_C"])]
    log_want = [k["SQRT2"], *reversed(k["LOG_B"]), k["LN2_HI"], k["LN2_LO"]]
    assert _fn_constants(src, "exp_cw") == [_bits(v) for v in exp_want]
    assert _fn_constants(src, "log_at") == [_bits(v) for v in log_want]


def test_missing_library_raises_no_fallback(tmp_path):
    # the binding has no CPU path: with the library absent every call raises before doing
    # anything (run in a fresh interpreter, since this process has loaded the library)
    import subprocess
    import sys
    code = (
        "import torch, invariant_amd as bi\n"
        f"bi.LIB_PATH = {str(tmp_path / 'absent' / 'libbi.so')!r}\n"
        "x = torch.zeros((2, 8), dtype=torch.bfloat16)\n"
        "g = torch.ones(8, dtype=torch.bfloat16)\n"
        "for f in (lambda: bi.bi_rmsnorm(x, g, 1e-5), lambda: bi.bi_gemm(x, x)):\n"
        "    try:\n"
        "        f()\n"
        "    except RuntimeError as e:\n"
        "        assert 'not built' in str(e), e\n"
        "    else:\n"
        "        raise SystemExit('a call returned without the library')\n"
        "print('raised')\n")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0 and "raised" in r.stdout, (r.stdout, r.stderr)


def test_abi_from_plain_c(lib, tmp_path):
    # include/bi.h as C99 and libbi.so linked from a C program: configuration, status
    # strings and validation (tests/c/abi_from_c.c; no GPU work)
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    exe = str(tmp_path / "abi_from_c")
    libdir = os.path.dirname(bi.LIB_PATH)
    build = subprocess.run([cc, "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"),
                            os.path.join(ROOT, "tests", "c", "abi_from_c.c"), "-o", exe,
                            f"-L{libdir}", "-l:" + os.path.basename(bi.LIB_PATH), f"-Wl,-rpath,{libdir}"],
                           capture_output=True, text=True)
    assert build.returncode == 0, build.stderr
    run = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert run.returncode == 0 and run.stdout.strip() == "ok", (run.stdout, run.stderr)


def test_binding_rejects_mismatched_shapes():
    # host-side shape checks of the binding, raised before any pointer reaches the library:
    # a packed B whose tile grid does not match (N, K), and a fused q/k/v row of the wrong
    # width for bi_rope_kv_write
    import torch
    a = torch.zeros((2, 1024), dtype=torch.bfloat16)
    good = torch.zeros((4, 32, 64, 8), dtype=torch.bfloat16)          # N = 64, K = 1024
    for bad in (torch.zeros((4, 31, 64, 8), dtype=torch.bfloat16),    # too few K steps
                torch.zeros((4, 32, 64, 8), dtype=torch.float32),
                good.transpose(0, 1)):
        with pytest.raises(ValueError, match="packed B"):
            bi.bi_gemm(a, bad, b_layout=bi.BI_B_TILED, n=64)
        with pytest.raises(ValueError, match="packed B"):
            bi.bi_gemm_swiglu(a, bad, w_layout=bi.BI_B_TILED)
    with pytest.raises(ValueError, match="packed B"):
        bi.bi_gemm(a, good, b_layout=bi.BI_B_TILED, n=65)             # 5 row blocks needed
    kc = torch.zeros((2, 2, 16, 16, 8), dtype=torch.bfloat16)         # [P, Hkv, D/8, page, 8]
    vc = torch.zeros((2, 2, 128, 16), dtype=torch.bfloat16)           # [P, Hkv, D, page]
    bt = torch.zeros((1, 2), dtype=torch.int32)
    sl = torch.ones(1, dtype=torch.int32)
    qsl = torch.tensor([0, 1], dtype=torch.int32)
    with pytest.raises(ValueError, match="qkv rows"):
        bi.bi_rope_kv_write(torch.zeros((1, 7 * 128), dtype=torch.bfloat16), kc, vc, bt, sl, qsl, 4)
    with pytest.raises(ValueError, match="contiguous"):
        bi.bi_rope_kv_write(torch.zeros((1, 8 * 128), dtype=torch.bfloat16), kc, vc, bt, sl, qsl, 4,
                            q=torch.zeros((1, 4, 64), dtype=torch.bfloat16))
