"""The C-ABI library: it loads, exports every function include/nvfp4moe.h declares,
and rejects bad arguments on the host before anything reaches a GPU.

No call here passes a device pointer, so these run without a GPU.
"""
import ctypes
import os
import re

import pytest

import precision_moe_gemm_amd as pmg

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "nvfp4moe.h")

OK, ERR_NULL, ERR_SHAPE, ERR_ALIGN, ERR_WORKSPACE, ERR_LAUNCH, ERR_ARG, ERR_SCRATCH = range(8)


def declared_functions():
    text = open(HEADER).read()
    return re.findall(r"NVFP4MOE_API\s+[\w\s\*]+?\b(\w+)\s*\(", text)


def test_header_declares_the_entry_points():
    names = set(declared_functions())
    for n in ("nvfp4_quantize_permute", "nvfp4_grouped_gemm", "swiglu_quantize", "unpermute_combine",
              "nvfp4_quantize_rows", "bf16_grouped_gemm", "bf16_grouped_gemm_gather", "permute_gather_bf16",
              "swiglu_backward", "bf16_transpose"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert set(declared_functions()) == set(pmg.SIGNATURES)


def test_version_and_status_strings(lib):
    assert lib.nvfp4moe_abi_version() == 2
    for s in range(8):
        assert pmg.status_string(s) and pmg.status_string(s) != pmg.status_string(99)
    assert "unknown" in pmg.status_string(99)


def test_workspace_size(lib):
    # a (chunk of 2048 or 4096 entries, expert) count table and one rank per routing entry
    assert lib.nvfp4moe_permute_workspace_size(4096, 8, 128) >= (8 * 128 + 32768) * 4
    assert lib.nvfp4moe_permute_workspace_size(0, 8, 128) >= 128 * 4
    assert lib.nvfp4moe_permute_workspace_size(-1, 8, 128) == 0


FAKE = 0x100000  # a 16-byte aligned non-null value; never dereferenced (calls fail before any launch)


def test_quantize_rows_host_checks(lib):
    f = lib.nvfp4_quantize_rows
    assert f(FAKE, 4, 24, FAKE, FAKE, FAKE, None) == ERR_SHAPE        # K % 16
    assert f(FAKE, 4, 8208, FAKE, FAKE, FAKE, None) == ERR_SHAPE      # K too large
    assert f(FAKE, -1, 32, FAKE, FAKE, FAKE, None) == ERR_SHAPE
    assert f(None, 4, 32, FAKE, FAKE, FAKE, None) == ERR_NULL
    assert f(FAKE + 4, 4, 32, FAKE, FAKE, FAKE, None) == ERR_ALIGN
    assert f(None, 0, 32, None, None, None, None) == OK               # nothing to do


def test_quantize_permute_host_checks(lib):
    f = lib.nvfp4_quantize_permute
    ws = lib.nvfp4moe_permute_workspace_size(64, 8, 128)
    args = lambda **kw: [kw.get("x", FAKE), kw.get("T", 64), kw.get("H", 256), kw.get("ids", FAKE),
                         kw.get("k", 8), kw.get("E", 128), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                         kw.get("ws", FAKE), kw.get("wsb", ws), None, None]
    assert f(*args(k=9, E=8)) == ERR_SHAPE                  # k > E
    assert f(*args(k=0)) == ERR_SHAPE
    assert f(*args(k=33, E=64)) == ERR_SHAPE                # k above the supported maximum
    assert f(*args(E=2000)) == ERR_SHAPE
    assert f(*args(H=40)) == ERR_SHAPE                      # H % 16
    assert f(*args(ids=None)) == ERR_NULL
    assert f(*args(ws=None)) == ERR_NULL
    assert f(*args(wsb=ws - 1)) == ERR_WORKSPACE
    assert f(*args(x=FAKE + 8)) == ERR_ALIGN
    assert f(*args(T=1 << 27, k=8, wsb=1 << 40)) == ERR_SHAPE   # T k above INT32_MAX / 2


def test_quantize_permute_noalloc_host_checks(lib):
    f = lib.nvfp4_quantize_permute_noalloc
    big = (1 << 20) // 8 + 1                                # T * k one chunk past the scratch
    assert f(FAKE, big, 256, FAKE, 8, 128, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None) == ERR_SCRATCH
    assert f(FAKE, -1, 256, FAKE, 8, 128, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None) == ERR_SHAPE
    assert "scratch" in pmg.status_string(ERR_SCRATCH)


def test_gemm_host_checks(lib):
    f = lib.nvfp4_grouped_gemm
    base = dict(E=128, R=32768, N=1536, K=2048)
    call = lambda **kw: f(FAKE, FAKE, FAKE, FAKE, kw.get("E", 128), kw.get("R", 32768), FAKE, FAKE,
                          kw.get("wr", FAKE), kw.get("N", 1536), kw.get("K", 2048), kw.get("lay", 0),
                          kw.get("c", FAKE), kw.get("cd", 0), None)
    assert call(cd=2) == ERR_ARG                            # unknown output dtype
    assert call(K=2000) == ERR_SHAPE                        # K % 64
    assert call(N=(1 << 20) + 16) == ERR_SHAPE
    assert call(lay=2) == ERR_ARG
    assert call(N=1537) == ERR_SHAPE
    assert call(E=0) == ERR_SHAPE
    assert call(c=None) == ERR_NULL
    assert call(wr=FAKE + 4) == ERR_ALIGN
    g = lib.bf16_grouped_gemm
    assert g(FAKE, FAKE, 128, 32768, FAKE, 7, 768, 2048, FAKE, None) == ERR_ARG
    assert g(FAKE, FAKE, 128, 32768, FAKE, 0, 768, 2040, FAKE, None) == ERR_SHAPE
    gg = lib.bf16_grouped_gemm_gather
    #        a     T     map   k  offsets E    R_cap  w    lay N    K     c     stream
    assert gg(FAKE, 4096, FAKE, 0, FAKE, 128, 32768, FAKE, 0, 768, 2048, FAKE, None) == ERR_SHAPE
    assert gg(FAKE, 4096, FAKE, 33, FAKE, 128, 32768, FAKE, 0, 768, 2048, FAKE, None) == ERR_SHAPE
    assert gg(FAKE, 4096, None, 8, FAKE, 128, 32768, FAKE, 0, 768, 2048, FAKE, None) == ERR_NULL
    assert gg(FAKE, 0, FAKE, 8, FAKE, 128, 32768, FAKE, 0, 768, 2048, FAKE, None) == ERR_SHAPE
    assert gg(FAKE, 1 << 21, FAKE, 8, FAKE, 128, 32768, FAKE, 0, 768, 2048, FAKE, None) == ERR_SHAPE  # 4 GiB
    assert gg(FAKE, 4096, FAKE, 8, FAKE, 128, 32768, FAKE, 3, 768, 2048, FAKE, None) == ERR_ARG
    assert gg(FAKE + 4, 4096, FAKE, 8, FAKE, 128, 32768, FAKE, 0, 768, 2048, FAKE, None) == ERR_ALIGN
    assert gg(None, 0, None, 8, None, 128, 0, None, 0, 768, 2048, None, None) == OK


def test_quantize_rows_tiled_host_checks(lib):
    f = lib.nvfp4_quantize_rows_tiled
    assert f(FAKE, 8, 96, 4, FAKE, FAKE, FAKE, None) == ERR_SHAPE     # K % 64
    assert f(FAKE, 8, 128, 3, FAKE, FAKE, FAKE, None) == ERR_SHAPE    # rows % group_rows
    assert f(FAKE, 8, 128, 0, FAKE, FAKE, FAKE, None) == ERR_SHAPE
    assert f(None, 8, 128, 4, FAKE, FAKE, FAKE, None) == ERR_NULL
    assert f(FAKE, 8, 128, 4, FAKE + 4, FAKE, FAKE, None) == ERR_ALIGN
    assert f(None, 0, 128, 4, None, None, None, None) == OK


def test_streaming_ops_host_checks(lib):
    assert lib.swiglu_quantize(FAKE, 100, 40, FAKE, 4, None, None, FAKE, FAKE, FAKE, None, None) == ERR_SHAPE
    assert lib.swiglu_quantize(FAKE, 100, 64, FAKE, 4, FAKE, None, FAKE, FAKE, FAKE, None, None) == ERR_NULL
    assert lib.unpermute_combine(FAKE, 10, 8, 2044, FAKE, None, FAKE, None) == ERR_SHAPE
    assert lib.unpermute_combine(FAKE, 10, 8, 2048, None, None, FAKE, None) == ERR_NULL
    assert lib.permute_gather_bf16(FAKE, 10, 2048, 8, FAKE, 0, FAKE, FAKE, None) == ERR_SHAPE
    assert lib.swiglu_backward(FAKE, FAKE, 10, 768, FAKE, 4, None, None, FAKE + 2, None) == ERR_ALIGN


def test_transpose_host_checks(lib):
    assert lib.bf16_transpose(FAKE, 2, 12, 16, FAKE + 64, None) == ERR_SHAPE        # rows % 8
    assert lib.bf16_transpose(FAKE, 65536, 8, 8, FAKE + 64, None) == ERR_SHAPE      # too many matrices
    assert lib.bf16_transpose(FAKE, 1, 65536, 65536, FAKE + 64, None) == ERR_SHAPE  # rows * cols > INT32_MAX
    assert lib.bf16_transpose(None, 0, 8, 8, None, None) == OK                      # nothing to do
    assert lib.bf16_transpose(None, 1, 8, 8, FAKE, None) == ERR_NULL
    assert lib.bf16_transpose(FAKE + 2, 1, 8, 8, FAKE + 64, None) == ERR_ALIGN
    assert lib.bf16_transpose(FAKE, 1, 8, 8, FAKE, None) == ERR_ARG                 # in place


def test_mfma_ceiling_host_checks(lib):
    assert lib.nvfp4moe_mfma_ceiling(0, None, None) == ERR_SHAPE
    assert lib.nvfp4moe_mfma_ceiling(10_000_001, None, None) == ERR_SHAPE
    assert lib.nvfp4moe_mfma_ceiling(10, None, None) == ERR_NULL
    assert lib.nvfp4moe_mfma_ceiling(10, 8, None) == ERR_ALIGN


def test_binding_raises_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(pmg, "_LIB", None)
    monkeypatch.setattr(pmg, "library_path", lambda: str(tmp_path / "missing.so"))
    with pytest.raises(pmg.LibraryNotBuilt):
        pmg.load_library()


def test_workspace_size_by_op(lib):
    T, k, E = 4096, 8, 128
    assert pmg.workspace_size(pmg.OP_QUANTIZE_PERMUTE, T=T, E=E, k=k) == lib.nvfp4moe_permute_workspace_size(T, k, E)
    for op in (pmg.OP_QUANTIZE_ROWS, pmg.OP_GROUPED_GEMM, pmg.OP_SWIGLU_QUANTIZE, pmg.OP_UNPERMUTE_COMBINE,
               pmg.OP_BF16_GROUPED_GEMM, pmg.OP_SWIGLU_BACKWARD):
        assert pmg.workspace_size(op, T=T, E=E, k=k, R_max=T * k, N=1536) == 0
    assert pmg.workspace_size(99) == 2 ** 64 - 1


def test_scale_and_code_indices_match_the_layouts():
    """The exported index functions against the layouts stated in the header: the
    row-major layout is [rows][K/16] / [rows][K/2]; the K-tiled layout moves the
    same bytes to [rows/G][K/64][G][4] / [rows/G][K/64][G][32].  Built here by
    numpy reshapes of an array of byte labels, independent of the C functions."""
    import numpy as np
    for rows, K, G in [(6, 128, 3), (8, 64, 8), (4, 192, 1)]:
        lab_s = np.arange(rows * K // 16).reshape(rows, K // 16)        # row-major: label = offset
        lab_c = np.arange(rows * K // 2).reshape(rows, K // 2)
        til_s = lab_s.reshape(rows // G, G, K // 64, 4).transpose(0, 2, 1, 3).reshape(-1)
        til_c = lab_c.reshape(rows // G, G, K // 64, 32).transpose(0, 2, 1, 3).reshape(-1)
        pos_s = np.empty_like(til_s); pos_s[til_s] = np.arange(til_s.size)   # label -> K-tiled offset
        pos_c = np.empty_like(til_c); pos_c[til_c] = np.arange(til_c.size)
        for r in range(rows):
            for kb in range(K // 16):
                assert pmg.bscale_index(r, kb, K) == lab_s[r, kb]
                assert pmg.bscale_index(r, kb, K, G) == pos_s[lab_s[r, kb]]
            for i in range(K):
                assert pmg.code_index(r, i, K) == lab_c[r, i // 2]
                assert pmg.code_index(r, i, K, G) == pos_c[lab_c[r, i // 2]]
    assert pmg.bscale_index(0, 8, 128) == -1 and pmg.code_index(0, 128, 128) == -1
    assert pmg.bscale_index(0, 0, 96, 4) == -1                         # K-tiled needs K % 64


def test_fused_swiglu_host_checks(lib):
    f = lib.nvfp4_grouped_gemm_swiglu
    #            A                      off   E    R_cap  W                  I    K     topk_w map   h     gu    ws    wsb     stream
    call = lambda **kw: f(FAKE, FAKE, FAKE, FAKE, 128, 32768, FAKE, FAKE, FAKE, kw.get("I", 768), 2048,
                          kw.get("tw", FAKE), kw.get("map", FAKE), FAKE, None, kw.get("ws", FAKE),
                          kw.get("wsb", 32768 * 4), None)
    assert call(I=640) == ERR_SHAPE                         # I % 256
    assert call(map=None) == ERR_NULL                       # router weights need the row map
    assert call(ws=None) == ERR_NULL
    assert call(wsb=32768 * 4 - 1) == ERR_WORKSPACE
    assert pmg.workspace_size(pmg.OP_GROUPED_GEMM_SWIGLU, R_max=32768) == 32768 * 4
    q = lib.nvfp4_quantize_rows_f32
    assert q(FAKE, 4, 24, None, 0, FAKE, FAKE, FAKE, None) == ERR_SHAPE
    assert q(FAKE, 4, 32, FAKE, 0, FAKE, FAKE, FAKE, None) == ERR_SHAPE   # offsets with E = 0
    assert q(FAKE + 4, 4, 32, None, 0, FAKE, FAKE, FAKE, None) == ERR_ALIGN
