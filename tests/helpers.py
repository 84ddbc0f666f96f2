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
    """Row-major NVFP4 [G, R, K/2] / [G, R, K/16] -> the K-tiled layout
    [G, K/64, R, 32] / [G, K/64, R, 4] (a pure move of bytes)."""
    G, R, half = codes.shape
    kt = half // 32
    return (codes.reshape(G, R, kt, 32).transpose(0, 2, 1, 3).copy(),
            bscales.reshape(G, R, kt, 4).transpose(0, 2, 1, 3).copy())


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
    """True where x lies within rel*|x| of a bf16 rounding midpoint (neighbours from the bit pattern)."""
    b = of.round_to_bf16(x64).astype(np.int32)
    mag = b & 0x7FFF
    sign = b & 0x8000
    q = of.bf16_to_f32(b.astype(np.uint16)).astype(np.float64)
    up = of.bf16_to_f32((sign | np.minimum(mag + 1, 0x7F7F)).astype(np.uint16)).astype(np.float64)
    dn = of.bf16_to_f32((sign | np.maximum(mag - 1, 0)).astype(np.uint16)).astype(np.float64)
    dist = np.minimum(np.abs(x64 - (q + up) / 2), np.abs(x64 - (q + dn) / 2))
    return dist <= rel * np.maximum(np.abs(x64), 1e-300)


class BF16Experts:
    """Per-expert float32 view of bf16 expert weights [E, ...] for the oracle's
    bf16 GEMM, converted only for the experts it touches (the whole tensor
    would not fit host memory in float)."""

    def __init__(self, bits):
        self.bits = bits
        self.shape = bits.shape

    def __getitem__(self, e):
        return of.bf16_to_f32(self.bits[e])
