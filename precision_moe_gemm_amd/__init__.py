"""MI355X (gfx950) NVFP4 W4A4 MoE hot path: a thin Python binding over libnvfp4moe.so.

Every function here marshals arguments into the C ABI declared in
``include/nvfp4moe.h`` and calls it on the current HIP stream; all arithmetic
runs in the library's HIP kernels.  PyTorch supplies device memory and the
stream only.  If the library has not been built, calls raise
``LibraryNotBuilt`` - there is no fallback implementation.

Tensor conventions: bf16 data may be passed as ``torch.bfloat16`` or as
2-byte integer tensors holding the bits; NVFP4 codes and scales are
``torch.uint8``; row scales, GEMM outputs and router weights ``torch.float32``;
routing ids, offsets and identity maps ``torch.int32``.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB = None

W_KN = 0
W_NK = 1
W_ROWMAJOR = 0   # NVFP4 weights [E, N, K/2] / [E, N, K/16]
W_KTILED = 1     # NVFP4 weights [E, K/64, N, 32] / [E, K/64, N, 4]
OUT_F32 = 0      # grouped GEMM output dtypes
OUT_BF16 = 1
OP_QUANTIZE_PERMUTE, OP_QUANTIZE_ROWS, OP_GROUPED_GEMM, OP_SWIGLU_QUANTIZE = 0, 1, 2, 3
OP_UNPERMUTE_COMBINE, OP_BF16_GROUPED_GEMM, OP_SWIGLU_BACKWARD, OP_GROUPED_GEMM_SWIGLU = 4, 5, 6, 7


class LibraryNotBuilt(RuntimeError):
    pass


class NVFP4Error(RuntimeError):
    def __init__(self, fn: str, status: int, text: str):
        super().__init__(f"{fn} failed with status {status}: {text}")
        self.status = status


def library_path() -> str:
    return os.path.join(_PKG, "libnvfp4moe.so")


_c = ctypes
_P = _c.c_void_p
_I64 = _c.c_int64
_I32 = _c.c_int32

# C signatures, in the order of include/nvfp4moe.h
SIGNATURES = {
    "nvfp4moe_status_string": ([_I32], _c.c_char_p),
    "nvfp4moe_abi_version": ([], _c.c_int),
    "nvfp4moe_permute_workspace_size": ([_I64, _I32, _I32], _c.c_size_t),
    "nvfp4moe_workspace_size": ([_I32, _I64, _I32, _I32, _I64, _I64], _c.c_size_t),
    "nvfp4moe_bscale_index": ([_I64, _I64, _I64, _I64], _I64),
    "nvfp4moe_code_index": ([_I64, _I64, _I64, _I64], _I64),
    "nvfp4_quantize_rows": ([_P, _I64, _I64, _P, _P, _P, _P], _c.c_int),
    "nvfp4_quantize_permute": ([_P, _I64, _I64, _P, _I32, _I32, _P, _P, _P, _P, _P, _P, _P,
                                _c.c_size_t, _P, _P], _c.c_int),
    "nvfp4_quantize_permute_noalloc": ([_P, _I64, _I64, _P, _I32, _I32, _P, _P, _P, _P, _P, _P, _P, _P],
                                       _c.c_int),
    "nvfp4_quantize_rows_tiled": ([_P, _I64, _I64, _I64, _P, _P, _P, _P], _c.c_int),
    "nvfp4_grouped_gemm": ([_P, _P, _P, _P, _I32, _I64, _P, _P, _P, _I64, _I64, _I32, _P, _I32, _P],
                           _c.c_int),
    "nvfp4_grouped_gemm_swiglu": ([_P, _P, _P, _P, _I32, _I64, _P, _P, _P, _I64, _I64, _P, _P, _P, _P, _P,
                                   _c.c_size_t, _P], _c.c_int),
    "nvfp4_quantize_rows_f32": ([_P, _I64, _I64, _P, _I32, _P, _P, _P, _P], _c.c_int),
    "nvfp4moe_token_blocks": ([_P, _I32, _P, _P], _c.c_int),
    "nvfp4_quantize_tokens": ([_P, _I32, _I64, _I64, _P, _I32, _P, _P, _I32, _I64, _I32, _P, _P, _P, _P],
                              _c.c_int),
    "nvfp4_grouped_gemm_wgrad": ([_P, _P, _P, _P, _P, _P, _P, _I32, _I64, _I64, _I64, _P, _I32, _P], _c.c_int),
    "swiglu_quantize": ([_P, _I64, _I64, _P, _I32, _P, _P, _P, _P, _P, _P, _P], _c.c_int),
    "unpermute_combine": ([_P, _I64, _I32, _I64, _P, _P, _P, _P], _c.c_int),
    "permute_gather_bf16": ([_P, _I64, _I64, _I32, _P, _I32, _P, _P, _P], _c.c_int),
    "bf16_grouped_gemm": ([_P, _P, _I32, _I64, _P, _I32, _I64, _I64, _P, _P], _c.c_int),
    "bf16_grouped_gemm_gather": ([_P, _I64, _P, _I32, _P, _I32, _I64, _P, _I32, _I64, _I64, _P, _P],
                                 _c.c_int),
    "swiglu_backward": ([_P, _P, _I64, _I64, _P, _I32, _P, _P, _P, _P], _c.c_int),
    "bf16_transpose": ([_P, _I64, _I64, _I64, _P, _P], _c.c_int),
    "nvfp4moe_mfma_ceiling": ([_I64, _P, _P], _c.c_int),
}


def load_library():
    """Load libnvfp4moe.so (cached).  Raises LibraryNotBuilt if it is missing."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = library_path()
    if not os.path.exists(path):
        raise LibraryNotBuilt(
            f"{path} is missing: build it with `python -m precision_moe_gemm_amd.build`")
    lib = ctypes.CDLL(path)
    for name, (args, res) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _LIB = lib
    return lib


def status_string(status: int) -> str:
    return load_library().nvfp4moe_status_string(status).decode()


def _check(fn: str, status: int):
    if status != 0:
        raise NVFP4Error(fn, status, status_string(status))


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _req(t, name, dtypes, ndim=None, numel=None):
    """Check a tensor argument; `numel`: the elements the library reads or writes
    through it (the C-ABI sees only the pointer, so a smaller buffer is refused here)."""
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name}: dtype {t.dtype} not in {dtypes}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {t.dim()}")
    if numel is not None and t.numel() < numel:
        raise ValueError(f"{name} holds {t.numel()} elements, needs {numel}")


_BF16 = (torch.bfloat16, torch.int16, torch.uint16)
_U8 = (torch.uint8,)
_F32 = (torch.float32,)
_I32T = (torch.int32,)


def _empty(shape, dtype, like):
    return torch.empty(shape, dtype=dtype, device=like.device)


# ---------------------------------------------------------------------- entry points
def nvfp4_quantize_rows(x, codes=None, bscales=None, rscales=None):
    """x bf16 [rows, K] -> (codes u8 [rows, K/2], bscales u8 [rows, K/16], rscales f32 [rows])."""
    _req(x, "x", _BF16, 2)
    rows, K = x.shape
    codes = _empty((rows, K // 2), torch.uint8, x) if codes is None else codes
    bscales = _empty((rows, K // 16), torch.uint8, x) if bscales is None else bscales
    rscales = _empty((rows,), torch.float32, x) if rscales is None else rscales
    _req(codes, "codes", _U8, numel=rows * (K // 2)); _req(bscales, "bscales", _U8, numel=rows * (K // 16))
    _req(rscales, "rscales", _F32, numel=rows)
    _check("nvfp4_quantize_rows", load_library().nvfp4_quantize_rows(
        _ptr(x), rows, K, _ptr(codes), _ptr(bscales), _ptr(rscales), _stream()))
    return codes, bscales, rscales


def nvfp4_quantize_rows_tiled(x, group_rows: int, codes=None, bscales=None, rscales=None):
    """x bf16 [rows, K] -> the K-tiled NVFP4 layout of groups of `group_rows` rows:
    (codes u8 [rows/G, K/64, G, 32], bscales u8 [rows/G, K/64, G, 4], rscales f32 [rows])."""
    _req(x, "x", _BF16, 2)
    rows, K = x.shape
    G = int(group_rows)
    if G <= 0 or rows % G or K % 64:
        raise ValueError("need rows % group_rows == 0 and K % 64 == 0")
    codes = _empty((rows // G, K // 64, G, 32), torch.uint8, x) if codes is None else codes
    bscales = _empty((rows // G, K // 64, G, 4), torch.uint8, x) if bscales is None else bscales
    rscales = _empty((rows,), torch.float32, x) if rscales is None else rscales
    _req(codes, "codes", _U8, numel=rows * (K // 2)); _req(bscales, "bscales", _U8, numel=rows * (K // 16))
    _req(rscales, "rscales", _F32, numel=rows)
    _check("nvfp4_quantize_rows_tiled", load_library().nvfp4_quantize_rows_tiled(
        _ptr(x), rows, K, G, _ptr(codes), _ptr(bscales), _ptr(rscales), _stream()))
    return codes, bscales, rscales


def permute_workspace_size(T: int, k: int, E: int) -> int:
    return int(load_library().nvfp4moe_permute_workspace_size(T, k, E))


def workspace_size(op: int, T: int = 0, E: int = 0, k: int = 0, R_max: int = 0, N: int = 0) -> int:
    """Device workspace bytes of an operation (OP_*); only OP_QUANTIZE_PERMUTE needs any."""
    return int(load_library().nvfp4moe_workspace_size(op, T, E, k, R_max, N))


def bscale_index(r: int, kb: int, K: int, group_rows: int = 0) -> int:
    """Byte offset of block kb of row r: row-major (group_rows 0) or K-tiled groups."""
    return int(load_library().nvfp4moe_bscale_index(r, kb, K, group_rows))


def code_index(r: int, i: int, K: int, group_rows: int = 0) -> int:
    """Byte offset of the byte holding element i of row r (low nibble for even i)."""
    return int(load_library().nvfp4moe_code_index(r, i, K, group_rows))


def nvfp4_quantize_permute(x, topk_ids, E: int, workspace=None, dev_err=None, out=None):
    """Route + permute + quantise.  Returns dict with codes, bscales, rscales,
    expert_offsets [E+1], row_to_tk [T*k], tk_to_row [T*k]."""
    _req(x, "x", _BF16, 2)
    _req(topk_ids, "topk_ids", _I32T, 2)
    T, H = x.shape
    k = topk_ids.shape[1]
    if topk_ids.shape[0] != T:
        raise ValueError("topk_ids must have one row per token")
    R = T * k
    o = out or {}
    shapes = {"codes": ((R, H // 2), torch.uint8), "bscales": ((R, H // 16), torch.uint8),
              "rscales": ((R,), torch.float32), "expert_offsets": ((E + 1,), torch.int32),
              "row_to_tk": ((R,), torch.int32), "tk_to_row": ((R,), torch.int32)}
    res = {n: o[n] if n in o else _empty(shp, dt, x) for n, (shp, dt) in shapes.items()}
    ws_bytes = permute_workspace_size(T, k, E)
    if ws_bytes == 0:
        raise ValueError("invalid routing shape")
    if workspace is None:
        workspace = _empty((max(ws_bytes, 256),), torch.uint8, x)
    for name, (shp, _) in shapes.items():
        _req(res[name], name, _U8 if name in ("codes", "bscales") else _F32 if name == "rscales" else _I32T,
             numel=math.prod(shp))
    _req(workspace, "workspace", _U8)
    _req(dev_err, "dev_err", _I32T, numel=1)
    _check("nvfp4_quantize_permute", load_library().nvfp4_quantize_permute(
        _ptr(x), T, H, _ptr(topk_ids), k, E, _ptr(res["codes"]), _ptr(res["bscales"]),
        _ptr(res["rscales"]), _ptr(res["expert_offsets"]), _ptr(res["row_to_tk"]),
        _ptr(res["tk_to_row"]), _ptr(workspace), workspace.numel(), _ptr(dev_err), _stream()))
    return res


NOALLOC_MAX_ENTRIES = 1 << 20
_QP_OUTPUTS = ("codes", "bscales", "rscales", "expert_offsets", "row_to_tk", "tk_to_row")


def nvfp4_quantize_permute_noalloc(x, topk_ids, E: int, out, dev_err=None):
    """nvfp4_quantize_permute without a workspace and without any allocation: the
    library's fixed device scratch serves T*k <= NOALLOC_MAX_ENTRIES entries.  Every
    output must be given in `out` (same names and sizes as nvfp4_quantize_permute's
    result); returns `out`.  Calls on one device that overlap in time race."""
    _req(x, "x", _BF16, 2)
    _req(topk_ids, "topk_ids", _I32T, 2)
    T, H = x.shape
    k = topk_ids.shape[1]
    if topk_ids.shape[0] != T:
        raise ValueError("topk_ids must have one row per token")
    missing = [n for n in _QP_OUTPUTS if n not in out]
    if missing:
        raise ValueError(f"the allocation-free call needs every output given: missing {missing}")
    R = T * k
    need = {"codes": (R * (H // 2), _U8), "bscales": (R * (H // 16), _U8), "rscales": (R, _F32),
            "expert_offsets": (E + 1, _I32T), "row_to_tk": (R, _I32T), "tk_to_row": (R, _I32T)}
    for name, (n, dt) in need.items():
        _req(out[name], name, dt, numel=n)
    _req(dev_err, "dev_err", _I32T, numel=1)
    _check("nvfp4_quantize_permute_noalloc", load_library().nvfp4_quantize_permute_noalloc(
        _ptr(x), T, H, _ptr(topk_ids), k, E, _ptr(out["codes"]), _ptr(out["bscales"]),
        _ptr(out["rscales"]), _ptr(out["expert_offsets"]), _ptr(out["row_to_tk"]),
        _ptr(out["tk_to_row"]), _ptr(dev_err), _stream()))
    return out


def nvfp4_grouped_gemm(a_codes, a_bscales, a_rscales, expert_offsets, w_codes, w_bscales,
                       w_rscales, c=None, out_dtype=None):
    """C[r] = A[r] W_e^T over expert-grouped rows.  Returns C [R_cap, N], float32
    (default) or bfloat16 (out_dtype=torch.bfloat16, or a bf16 `c`).
    W in either layout: row-major codes [E, N, K/2] (bscales [E, N, K/16]) or
    K-tiled codes [E, K/64, N, 32] (bscales [E, K/64, N, 4]); w_rscales [E, N]."""
    for t, n, d in ((a_codes, "a_codes", _U8), (a_bscales, "a_bscales", _U8),
                    (a_rscales, "a_rscales", _F32), (expert_offsets, "expert_offsets", _I32T),
                    (w_codes, "w_codes", _U8), (w_bscales, "w_bscales", _U8),
                    (w_rscales, "w_rscales", _F32)):
        _req(t, n, d)
    R_cap = a_codes.shape[0]
    K = a_codes.shape[1] * 2
    E = expert_offsets.numel() - 1
    if w_codes.dim() == 4:
        layout, N = W_KTILED, w_codes.shape[2]
        ok = tuple(w_codes.shape) == (E, K // 64, N, 32) and tuple(w_bscales.shape) == (E, K // 64, N, 4)
    else:
        layout, N = W_ROWMAJOR, w_codes.shape[1]
        ok = (w_codes.dim() == 3 and w_codes.shape[0] == E and w_codes.shape[2] * 2 == K
              and w_bscales.numel() >= E * N * (K // 16))
    if not ok:
        raise ValueError("w_codes/w_bscales shapes do not match E, K and a known layout")
    _req(a_bscales, "a_bscales", _U8, numel=R_cap * (K // 16))
    _req(a_rscales, "a_rscales", _F32, numel=R_cap)
    _req(w_rscales, "w_rscales", _F32, numel=E * N)
    if out_dtype is None:
        out_dtype = torch.float32 if c is None or c.dtype == torch.float32 else torch.bfloat16
    if out_dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("out_dtype must be torch.float32 or torch.bfloat16")
    c = _empty((R_cap, N), out_dtype, a_codes) if c is None else c
    _req(c, "c", _F32 if out_dtype == torch.float32 else _BF16, numel=R_cap * N)
    _check("nvfp4_grouped_gemm", load_library().nvfp4_grouped_gemm(
        _ptr(a_codes), _ptr(a_bscales), _ptr(a_rscales), _ptr(expert_offsets), E, R_cap,
        _ptr(w_codes), _ptr(w_bscales), _ptr(w_rscales), N, K, layout, _ptr(c),
        OUT_F32 if out_dtype == torch.float32 else OUT_BF16, _stream()))
    return c


def nvfp4_grouped_gemm_swiglu(a_codes, a_bscales, a_rscales, expert_offsets, w_codes, w_bscales,
                              w_rscales, topk_w=None, row_to_tk=None, h=None, gu=None, want_gu=False,
                              workspace=None):
    """gate_up GEMM with the weighted SwiGLU in its epilogue.  W K-tiled
    (codes [E, K/64, 2I, 32], bscales [E, K/64, 2I, 4], rscales [E, 2I]).
    Returns (h f32 [R_cap, I], gu f32 [R_cap, 2I] or None)."""
    for t, n, d in ((a_codes, "a_codes", _U8), (a_bscales, "a_bscales", _U8),
                    (a_rscales, "a_rscales", _F32), (expert_offsets, "expert_offsets", _I32T),
                    (w_codes, "w_codes", _U8), (w_bscales, "w_bscales", _U8),
                    (w_rscales, "w_rscales", _F32), (topk_w, "topk_w", _F32), (row_to_tk, "row_to_tk", _I32T)):
        _req(t, n, d)
    R_cap = a_codes.shape[0]
    K = a_codes.shape[1] * 2
    E = expert_offsets.numel() - 1
    if w_codes.dim() != 4 or w_codes.shape[0] != E or w_codes.shape[1] != K // 64 or w_codes.shape[2] % 2:
        raise ValueError("w_codes must be K-tiled [E, K/64, 2I, 32]")
    N = w_codes.shape[2]
    I = N // 2
    if tuple(w_bscales.shape) != (E, K // 64, N, 4):
        raise ValueError("w_bscales must be K-tiled [E, K/64, 2I, 4]")
    _req(a_bscales, "a_bscales", _U8, numel=R_cap * (K // 16))
    _req(a_rscales, "a_rscales", _F32, numel=R_cap)
    _req(w_rscales, "w_rscales", _F32, numel=E * N)
    if topk_w is not None:
        if row_to_tk is None:
            raise ValueError("topk_w needs row_to_tk")
        _req(topk_w, "topk_w", _F32, numel=R_cap)
        _req(row_to_tk, "row_to_tk", _I32T, numel=R_cap)
        ws_bytes = workspace_size(OP_GROUPED_GEMM_SWIGLU, R_max=R_cap)
        workspace = _empty((ws_bytes,), torch.uint8, a_codes) if workspace is None else workspace
        _req(workspace, "workspace", _U8, numel=ws_bytes)
    h = _empty((R_cap, I), torch.float32, a_codes) if h is None else h
    _req(h, "h", _F32, numel=R_cap * I)
    if want_gu and gu is None:
        gu = _empty((R_cap, N), torch.float32, a_codes)
    _req(gu, "gu", _F32, numel=R_cap * N)
    _check("nvfp4_grouped_gemm_swiglu", load_library().nvfp4_grouped_gemm_swiglu(
        _ptr(a_codes), _ptr(a_bscales), _ptr(a_rscales), _ptr(expert_offsets), E, R_cap, _ptr(w_codes),
        _ptr(w_bscales), _ptr(w_rscales), I, K, _ptr(topk_w), _ptr(row_to_tk), _ptr(h), _ptr(gu),
        _ptr(workspace), 0 if workspace is None else workspace.numel(), _stream()))
    return h, gu


def nvfp4_quantize_rows_f32(x, expert_offsets=None, codes=None, bscales=None, rscales=None):
    """FP32 rows [rows, K] -> NVFP4 (codes, bscales, rscales); with expert_offsets only
    the routed rows [0, offsets[E]) are written."""
    _req(x, "x", _F32, 2)
    _req(expert_offsets, "expert_offsets", _I32T)
    rows, K = x.shape
    E = 0 if expert_offsets is None else expert_offsets.numel() - 1
    codes = _empty((rows, K // 2), torch.uint8, x) if codes is None else codes
    bscales = _empty((rows, K // 16), torch.uint8, x) if bscales is None else bscales
    rscales = _empty((rows,), torch.float32, x) if rscales is None else rscales
    _req(codes, "codes", _U8, numel=rows * (K // 2)); _req(bscales, "bscales", _U8, numel=rows * (K // 16))
    _req(rscales, "rscales", _F32, numel=rows)
    _check("nvfp4_quantize_rows_f32", load_library().nvfp4_quantize_rows_f32(
        _ptr(x), rows, K, _ptr(expert_offsets), E, _ptr(codes), _ptr(bscales), _ptr(rscales), _stream()))
    return codes, bscales, rscales


def token_blocks(expert_offsets, kofs=None):
    """kofs [E+1] int32: the first 64-token step of each expert's slab along K."""
    _req(expert_offsets, "expert_offsets", _I32T)
    E = expert_offsets.numel() - 1
    kofs = _empty((E + 1,), torch.int32, expert_offsets) if kofs is None else kofs
    _req(kofs, "kofs", _I32T, numel=E + 1)
    _check("nvfp4moe_token_blocks", load_library().nvfp4moe_token_blocks(
        _ptr(expert_offsets), E, _ptr(kofs), _stream()))
    return kofs


def token_capacity(R: int, E: int) -> int:
    """K positions that always hold every expert's padded slab."""
    return 64 * (-(-R // 64) + E)


def nvfp4_quantize_tokens(x, expert_offsets, kofs, Kp: int, layout: int = W_ROWMAJOR, row_to_tk=None, k: int = 1,
                          out=None):
    """Quantise along tokens, per expert: x [rows, C] (bf16 or f32; token order with
    row_to_tk/k, else expert-grouped rows).  Returns (codes, bscales, rscales [E, C]):
    row-major codes [C, Kp/2] / bscales [C, Kp/16], or K-tiled [Kp/64, C, 32] / [Kp/64, C, 4]."""
    _req(x, "x", _BF16 + _F32, 2)
    _req(expert_offsets, "expert_offsets", _I32T)
    _req(row_to_tk, "row_to_tk", _I32T)
    E = expert_offsets.numel() - 1
    _req(kofs, "kofs", _I32T, numel=E + 1)
    rows, C = x.shape
    if row_to_tk is None and rows < 1:
        raise ValueError("x has no rows")
    o = out or {}
    shp_c = (C, Kp // 2) if layout == W_ROWMAJOR else (Kp // 64, C, 32)
    shp_b = (C, Kp // 16) if layout == W_ROWMAJOR else (Kp // 64, C, 4)
    codes = o["codes"] if "codes" in o else _empty(shp_c, torch.uint8, x)
    bsc = o["bscales"] if "bscales" in o else _empty(shp_b, torch.uint8, x)
    rsc = o["rscales"] if "rscales" in o else _empty((E, C), torch.float32, x)
    _req(codes, "codes", _U8, numel=C * Kp // 2); _req(bsc, "bscales", _U8, numel=C * Kp // 16)
    _req(rsc, "rscales", _F32, numel=E * C)
    dt = 1 if x.dtype == torch.float32 else 0
    _check("nvfp4_quantize_tokens", load_library().nvfp4_quantize_tokens(
        _ptr(x), dt, rows, C, _ptr(row_to_tk), k, _ptr(expert_offsets), _ptr(kofs), E, Kp, layout,
        _ptr(codes), _ptr(bsc), _ptr(rsc), _stream()))
    return codes, bsc, rsc


def nvfp4_grouped_gemm_wgrad(a, w, kofs, c=None, out_dtype=None):
    """dW [E, M, N] = per expert dequant(A_e) dequant(W_e)^T over its token slab,
    float32 (default) or bfloat16 (out_dtype=torch.bfloat16, or a bf16 `c`).
    a: row-major (codes [M, Kp/2], bscales [M, Kp/16], rscales [E, M]);
    w: K-tiled (codes [Kp/64, N, 32], bscales [Kp/64, N, 4], rscales [E, N])."""
    ac, ab, ar = a
    wc, wb, wr = w
    for t, n, d in ((ac, "a_codes", _U8), (ab, "a_bscales", _U8), (ar, "a_rscales", _F32),
                    (wc, "w_codes", _U8), (wb, "w_bscales", _U8), (wr, "w_rscales", _F32), (kofs, "kofs", _I32T)):
        _req(t, n, d)
    M, half = ac.shape
    Kp = half * 2
    E = kofs.numel() - 1
    if wc.dim() != 3 or wc.shape[0] != Kp // 64 or wc.shape[2] != 32:
        raise ValueError("w codes must be K-tiled [Kp/64, N, 32] over the same Kp")
    N = wc.shape[1]
    _req(ab, "a_bscales", _U8, numel=M * Kp // 16); _req(ar, "a_rscales", _F32, numel=E * M)
    _req(wb, "w_bscales", _U8, numel=N * Kp // 16); _req(wr, "w_rscales", _F32, numel=E * N)
    if out_dtype is None:
        out_dtype = torch.float32 if c is None or c.dtype == torch.float32 else torch.bfloat16
    if out_dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("out_dtype must be torch.float32 or torch.bfloat16")
    c = _empty((E, M, N), out_dtype, ac) if c is None else c
    _req(c, "c", _F32 if out_dtype == torch.float32 else _BF16, numel=E * M * N)
    _check("nvfp4_grouped_gemm_wgrad", load_library().nvfp4_grouped_gemm_wgrad(
        _ptr(ac), _ptr(ab), _ptr(ar), _ptr(wc), _ptr(wb), _ptr(wr), _ptr(kofs), E, M, N, Kp, _ptr(c),
        OUT_F32 if out_dtype == torch.float32 else OUT_BF16, _stream()))
    return c


def swiglu_quantize(gu, expert_offsets, topk_w=None, row_to_tk=None, h_out=False, out=None):
    """Weighted SwiGLU + NVFP4 quantise of routed rows.  Returns (codes, bscales, rscales, h or None)."""
    _req(gu, "gu", _F32, 2)
    _req(expert_offsets, "expert_offsets", _I32T)
    _req(topk_w, "topk_w", _F32)
    _req(row_to_tk, "row_to_tk", _I32T)
    R_cap, I2 = gu.shape
    I = I2 // 2
    E = expert_offsets.numel() - 1
    # the kernel reads topk_w[row_to_tk[r]], and row_to_tk holds entries below R_cap
    _req(topk_w, "topk_w", _F32, numel=R_cap)
    o = out or {}
    codes = o["codes"] if "codes" in o else _empty((R_cap, I // 2), torch.uint8, gu)
    bsc = o["bscales"] if "bscales" in o else _empty((R_cap, I // 16), torch.uint8, gu)
    rsc = o["rscales"] if "rscales" in o else _empty((R_cap,), torch.float32, gu)
    h = (o["h"] if "h" in o else _empty((R_cap, I), torch.float32, gu)) if h_out else None
    _req(codes, "codes", _U8, numel=R_cap * (I // 2)); _req(bsc, "bscales", _U8, numel=R_cap * (I // 16))
    _req(rsc, "rscales", _F32, numel=R_cap); _req(h, "h", _F32, numel=R_cap * I)
    _req(row_to_tk, "row_to_tk", _I32T, numel=R_cap)
    _check("swiglu_quantize", load_library().swiglu_quantize(
        _ptr(gu), R_cap, I, _ptr(expert_offsets), E, _ptr(topk_w), _ptr(row_to_tk),
        _ptr(codes), _ptr(bsc), _ptr(rsc), _ptr(h), _stream()))
    return codes, bsc, rsc, h


def unpermute_combine(d, tk_to_row, k: int, topk_w=None, y=None):
    """y[t] = bf16(sum over slots of w * d[row(t, slot)]).  Returns y as torch.bfloat16 [T, H]."""
    _req(d, "d", _F32, 2)
    _req(tk_to_row, "tk_to_row", _I32T)
    _req(topk_w, "topk_w", _F32)
    if k < 1 or tk_to_row.numel() % k:
        raise ValueError("tk_to_row must hold T * k entries")
    T = tk_to_row.numel() // k
    H = d.shape[1]
    # tk_to_row names rows below T * k (the routed rows of nvfp4_quantize_permute)
    _req(d, "d", _F32, numel=T * k * H)
    _req(topk_w, "topk_w", _F32, numel=T * k)
    y = _empty((T, H), torch.bfloat16, d) if y is None else y
    _req(y, "y", _BF16, numel=T * H)
    _check("unpermute_combine", load_library().unpermute_combine(
        _ptr(d), T, k, H, _ptr(tk_to_row), _ptr(topk_w), _ptr(y), _stream()))
    return y


def permute_gather_bf16(x, expert_offsets, row_to_tk, k: int, out=None):
    _req(x, "x", _BF16, 2)
    _req(expert_offsets, "expert_offsets", _I32T)
    _req(row_to_tk, "row_to_tk", _I32T)
    T, H = x.shape
    E = expert_offsets.numel() - 1
    _req(row_to_tk, "row_to_tk", _I32T, numel=T * k)
    out = _empty((T * k, H), torch.bfloat16, x) if out is None else out
    _req(out, "out", _BF16, numel=T * k * H)
    _check("permute_gather_bf16", load_library().permute_gather_bf16(
        _ptr(x), T, H, k, _ptr(expert_offsets), E, _ptr(row_to_tk), _ptr(out), _stream()))
    return out


def bf16_transpose(x, out=None):
    """out[b] = x[b].T for bf16 x [B, rows, cols] (weight preparation).  Returns [B, cols, rows]."""
    _req(x, "x", _BF16, 3)
    B, rows, cols = x.shape
    out = _empty((B, cols, rows), torch.bfloat16, x) if out is None else out
    _req(out, "out", _BF16, numel=B * rows * cols)
    _check("bf16_transpose", load_library().bf16_transpose(_ptr(x), B, rows, cols, _ptr(out), _stream()))
    return out


def bf16_grouped_gemm(a, expert_offsets, w, w_layout: int = W_KN, c=None):
    """c[r] = a[r] @ W_e with W [E, K, N] (W_KN) or [E, N, K] (W_NK).  Returns f32 [R_cap, N]."""
    _req(a, "a", _BF16, 2)
    _req(expert_offsets, "expert_offsets", _I32T)
    _req(w, "w", _BF16, 3)
    R_cap, K = a.shape
    E = expert_offsets.numel() - 1
    N = w.shape[2] if w_layout == W_KN else w.shape[1]
    kw = w.shape[1] if w_layout == W_KN else w.shape[2]
    if kw != K or w.shape[0] != E:
        raise ValueError("weight shape does not match a / expert_offsets")
    c = _empty((R_cap, N), torch.float32, a) if c is None else c
    _req(c, "c", _F32, numel=R_cap * N)
    _check("bf16_grouped_gemm", load_library().bf16_grouped_gemm(
        _ptr(a), _ptr(expert_offsets), E, R_cap, _ptr(w), w_layout, N, K, _ptr(c), _stream()))
    return c


def bf16_grouped_gemm_gather(a, row_to_tk, k: int, expert_offsets, w, w_layout: int = W_KN, c=None):
    """c[r] = a[row_to_tk[r] // k] @ W_e: the grouped GEMM over token rows gathered in its loads.

    a bf16 [T, K]; row_to_tk int32 [R_cap].  Returns f32 [R_cap, N]."""
    _req(a, "a", _BF16, 2)
    _req(row_to_tk, "row_to_tk", _I32T)
    _req(expert_offsets, "expert_offsets", _I32T)
    _req(w, "w", _BF16, 3)
    T, K = a.shape
    R_cap = row_to_tk.numel()
    E = expert_offsets.numel() - 1
    N = w.shape[2] if w_layout == W_KN else w.shape[1]
    kw = w.shape[1] if w_layout == W_KN else w.shape[2]
    if kw != K or w.shape[0] != E:
        raise ValueError("weight shape does not match a / expert_offsets")
    c = _empty((R_cap, N), torch.float32, a) if c is None else c
    _req(c, "c", _F32, numel=R_cap * N)
    _check("bf16_grouped_gemm_gather", load_library().bf16_grouped_gemm_gather(
        _ptr(a), T, _ptr(row_to_tk), k, _ptr(expert_offsets), E, R_cap, _ptr(w), w_layout, N, K,
        _ptr(c), _stream()))
    return c


def swiglu_backward(gu, dh, expert_offsets, topk_w=None, row_to_tk=None, dgu=None):
    _req(gu, "gu", _F32, 2)
    _req(dh, "dh", _F32, 2)
    _req(expert_offsets, "expert_offsets", _I32T)
    _req(topk_w, "topk_w", _F32)
    _req(row_to_tk, "row_to_tk", _I32T)
    R_cap, I2 = gu.shape
    E = expert_offsets.numel() - 1
    _req(dh, "dh", _F32, numel=R_cap * (I2 // 2))
    _req(topk_w, "topk_w", _F32, numel=R_cap)
    _req(row_to_tk, "row_to_tk", _I32T, numel=R_cap)
    dgu = _empty((R_cap, I2), torch.bfloat16, gu) if dgu is None else dgu
    _req(dgu, "dgu", _BF16, numel=R_cap * I2)
    _check("swiglu_backward", load_library().swiglu_backward(
        _ptr(gu), _ptr(dh), R_cap, I2 // 2, _ptr(expert_offsets), E, _ptr(topk_w),
        _ptr(row_to_tk), _ptr(dgu), _stream()))
    return dgu


def mfma_ceiling(iters: int, sink=None):
    """Launch the FP16 MFMA-only measurement kernel on the current stream.

    Returns (sink, flops issued).  Timing is the caller's."""
    if sink is None:
        sink = torch.empty(256 * 512, dtype=torch.float32, device="cuda")
    _req(sink, "sink", _F32, numel=256 * 512)
    _check("nvfp4moe_mfma_ceiling", load_library().nvfp4moe_mfma_ceiling(iters, _ptr(sink), _stream()))
    return sink, 256 * 8 * iters * 8 * 32768
