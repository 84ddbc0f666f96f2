"""Helpers shared by the GPU parity tests (host <-> device copies and comparisons)."""
import numpy as np
import torch

import precision_moe_gemm_amd as pmg
from oracle import formats as of, quantize as oq

DEV = "cuda:0"


def gpu_ready():
    return torch.cuda.is_available()


def bf16_dev(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(DEV).view(torch.bfloat16)


def bf16_host(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy()


def quantize_weights_oracle(w_bits: np.ndarray, experts=None):
    """[E, N, K] bf16 bits -> oracle NVFP4 (codes [E,N,K/2], bscales [E,N,K/16], rscales [E,N]).

    With `experts`, only those experts are quantised (the others stay zero), so
    full-size checks on sampled rows need not quantise every expert on the CPU.
    """
    E, N, K = w_bits.shape
    c = np.zeros((E, N, K // 2), np.uint8)
    b = np.zeros((E, N, K // 16), np.uint8)
    s = np.zeros((E, N), np.float32)
    for e in (range(E) if experts is None else sorted(set(int(v) for v in experts))):
        c[e], b[e], s[e] = oq.quantize_rows_bf16(w_bits[e])
    return c, b, s


def quantize_weights_gpu(w_bits: np.ndarray):
    E, N, K = w_bits.shape
    c, b, s = pmg.nvfp4_quantize_rows(bf16_dev(w_bits.reshape(E * N, K)))
    return c.view(E, N, K // 2), b.view(E, N, K // 16), s.view(E, N)


def quantize_weights_gpu_tiled(w_bits: np.ndarray):
    """[E, N, K] bf16 bits -> K-tiled NVFP4 on the device (codes [E, K/64, N, 32],
    bscales [E, K/64, N, 4], rscales [E, N])."""
    E, N, K = w_bits.shape
    c, b, s = pmg.nvfp4_quantize_rows_tiled(bf16_dev(w_bits.reshape(E * N, K)), N)
    return c, b, s.view(E, N)


def ktile(codes: np.ndarray, bscales: np.ndarray):
    """Row-major NVFP4 [groups, G, K/2] / [groups, G, K/16] -> the K-tiled layout
    [groups, K/64, G, 32] / [groups, K/64, G, 4], each byte moved to the offset the
    library's nvfp4moe_code_index / nvfp4moe_bscale_index name for it.  The
    offsets of one group come from those functions (one call per byte); a later
    group's are the first group's plus the group's size, which is checked on
    the last group's first and last rows."""
    n_grp, G, half = codes.shape
    K = half * 2
    ci = np.array([[pmg.code_index(r, 2 * b, K, G) for b in range(half)] for r in range(G)], np.int64)
    si = np.array([[pmg.bscale_index(r, kb, K, G) for kb in range(K // 16)] for r in range(G)], np.int64)
    last = (n_grp - 1) * G
    for r in (0, G - 1):
        assert [pmg.code_index(last + r, 2 * b, K, G) for b in (0, half - 1)] == \
            [int(ci[r, 0]) + last * half, int(ci[r, -1]) + last * half]
        assert pmg.bscale_index(last + r, K // 16 - 1, K, G) == int(si[r, -1]) + last * (K // 16)
    out_c = np.empty(codes.size, np.uint8)
    out_s = np.empty(bscales.size, np.uint8)
    g_off = np.arange(n_grp, dtype=np.int64)[:, None, None]
    out_c[(ci[None] + g_off * G * half).reshape(-1)] = codes.reshape(-1)
    out_s[(si[None] + g_off * G * (K // 16)).reshape(-1)] = bscales.reshape(-1)
    return (out_c.reshape(n_grp, K // 64, G, 32), out_s.reshape(n_grp, K // 64, G, 4))


def assert_within(got: np.ndarray, ref: np.ndarray, bound: np.ndarray, what: str = ""):
    err = np.abs(got.astype(np.float64) - ref)
    bad = err > bound
    ratio = float((err / np.maximum(bound, 1e-300)).max()) if err.size else 0.0
    assert not bad.any(), (f"{what}: {int(bad.sum())} of {bad.size} elements outside the bound, "
                           f"worst err/bound {ratio:.3g}, first at {np.argwhere(bad)[:3].tolist()}")
    return ratio


def sample_rows(offsets: np.ndarray, experts, extra: int, seed: int):
    """All rows of the given experts plus `extra` more randomly chosen experts.

    Returns (rows sorted, experts used)."""
    rng = np.random.default_rng(seed)
    E = offsets.size - 1
    chosen = list(experts) + [int(e) for e in rng.choice(E, size=min(extra, E), replace=False)]
    rows = [np.arange(offsets[e], offsets[e + 1]) for e in chosen]
    return np.unique(np.concatenate(rows).astype(np.int64)), sorted(set(chosen))


def bf16_midpoint_adjacent(x64, rel=2.0 ** -40):
    """True where x lies within rel*|x| of a bf16 rounding midpoint (neighbours from the bit pattern);
    exact zeros are compared as they are, sign included."""
    b = of.round_to_bf16(x64).astype(np.int32)
    mag = b & 0x7FFF
    sign = b & 0x8000
    q = of.bf16_to_f32(b.astype(np.uint16)).astype(np.float64)
    up = of.bf16_to_f32((sign | np.minimum(mag + 1, 0x7F7F)).astype(np.uint16)).astype(np.float64)
    dn = of.bf16_to_f32((sign | np.maximum(mag - 1, 0)).astype(np.uint16)).astype(np.float64)
    dist = np.minimum(np.abs(x64 - (q + up) / 2), np.abs(x64 - (q + dn) / 2))
    # an exact zero is never near a midpoint (below, dn clamps to zero itself)
    return (dist <= rel * np.maximum(np.abs(x64), 1e-300)) & (x64 != 0)


class BF16Experts:
    """Per-expert float32 view of bf16 expert weights [E, ...] for the oracle's
    bf16 GEMM, converted only for the experts it touches (the whole tensor
    would not fit host memory in float)."""

    def __init__(self, bits):
        self.bits = bits
        self.shape = bits.shape

    def __getitem__(self, e):
        return of.bf16_to_f32(self.bits[e])
