"""Seeded synthetic inputs for the NVFP4 MoE hot path.

This module is shared by the tests, ``bench.py`` and ``__graft_entry__.smoke()``.
It holds none of the method's arithmetic: it draws random numbers, rounds them
to bf16 storage, and synthesises the router's choices (the host-side routing
that happens before the permutation the library performs).

Shapes follow a Qwen3-30B-A3B-like MoE layer (model named in the miniTE pages,
news.hamidun.com "miniTE accélère le RL en NVFP4 sur B300", §Paramètres clés):
hidden 2048, 128 experts, top-8, expert intermediate 768, sequence 4096
(the blog page "miniTE NVFP4", §Respect the timing boundaries, gives the
sequence length and micro-batch one).  No weights or datasets are used: every
tensor is synthetic and seeded with ``numpy.random.default_rng([config, tensor])``.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

# Layer shape (Qwen3-30B-A3B-like).
TOKENS = 4096
HIDDEN = 2048
EXPERTS = 128
TOPK = 8
INTER = 768
QKV_N = 5120  # 32 q heads + 2 x 4 kv heads, head dim 128

# Config ids used as the first seed word.
CFG_TINY, CFG_QPERM, CFG_GATEUP, CFG_DOWN, CFG_LAYER = 1, 2, 3, 4, 5


def rng(config: int, tensor: int) -> np.random.Generator:
    return np.random.default_rng([int(config), int(tensor)])


def f32_to_bf16_bits(x) -> np.ndarray:
    """Round float32 values to bf16 storage (nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(b) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def gaussian_bf16(shape, std: float, config: int, tensor: int) -> np.ndarray:
    g = rng(config, tensor).standard_normal(shape, dtype=np.float64) * std
    return f32_to_bf16_bits(g.astype(np.float32))


def activations(T: int, H: int, config: int, tensor: int = 0,
                outlier_frac: float = 0.01, outlier_scale: float = 20.0) -> np.ndarray:
    """bf16 activations ~N(0,1) with i.i.d. Bernoulli(outlier_frac) elements scaled by outlier_scale."""
    g = rng(config, tensor)
    x = g.standard_normal((T, H), dtype=np.float64)
    if outlier_frac > 0:
        mask = g.random((T, H)) < outlier_frac
        x = np.where(mask, x * outlier_scale, x)
    return f32_to_bf16_bits(x.astype(np.float32))


def router_logits(T: int, E: int, config: int, tensor: int = 1) -> np.ndarray:
    return rng(config, tensor).standard_normal((T, E), dtype=np.float64).astype(np.float32)


def route_softmax_topk(logits: np.ndarray, k: int):
    """Top-k of a softmax router: experts ordered by (logit desc, id asc); weights renormalised over the k.

    Returns (ids int32 [T,k], weights float32 [T,k]).
    """
    logits = np.asarray(logits, dtype=np.float32)
    order = np.argsort(-logits, axis=1, kind="stable")[:, :k]
    sel = np.take_along_axis(logits, order, axis=1).astype(np.float64)
    ex = np.exp(sel - sel[:, :1])
    w = ex / ex.sum(axis=1, keepdims=True)
    return order.astype(np.int32), w.astype(np.float32)


def _weights_for(ids: np.ndarray, config: int, tensor: int) -> np.ndarray:
    lg = rng(config, tensor).standard_normal(ids.shape, dtype=np.float64)
    ex = np.exp(lg - lg.max(axis=1, keepdims=True))
    return (ex / ex.sum(axis=1, keepdims=True)).astype(np.float32)


def route_uniform(T: int, E: int, k: int, config: int, tensor: int = 2):
    """A uniformly random k-subset of experts per token (random order within the token)."""
    keys = rng(config, tensor).random((T, E))
    ids = np.argsort(keys, axis=1, kind="stable")[:, :k].astype(np.int32)
    return ids, _weights_for(ids, config, tensor + 100)


def route_zipf(T: int, E: int, k: int, s: float, config: int, tensor: int = 3):
    """k distinct experts per token, Gumbel-top-k with p(e) proportional to (e+1)^-s (expert 0 most popular)."""
    logp = -s * np.log(np.arange(1, E + 1, dtype=np.float64))
    gum = rng(config, tensor).gumbel(size=(T, E))
    ids = np.argsort(-(logp[None, :] + gum), axis=1, kind="stable")[:, :k].astype(np.int32)
    return ids, _weights_for(ids, config, tensor + 100)


def make_routing(kind: str, T: int, E: int, k: int, config: int):
    if kind == "softmax":
        return route_softmax_topk(router_logits(T, E, config), k)
    if kind == "uniform":
        return route_uniform(T, E, k, config)
    if kind == "zipf":
        return route_zipf(T, E, k, 1.2, config)
    raise ValueError(f"unknown routing kind {kind!r}")


@dataclass(frozen=True)
class LayerShape:
    T: int = TOKENS
    H: int = HIDDEN
    E: int = EXPERTS
    k: int = TOPK
    I: int = INTER
    qkv_n: int = QKV_N

    @property
    def R(self) -> int:
        return self.T * self.k


def moe_weights_bf16(shape: LayerShape, config: int, std: float = 0.02):
    """bf16 master weights: W_gu [E][2I][H] (gate rows first, then up rows), W_d [E][H][I]."""
    w_gu = gaussian_bf16((shape.E, 2 * shape.I, shape.H), std, config, 10)
    w_d = gaussian_bf16((shape.E, shape.H, shape.I), std, config, 11)
    return w_gu, w_d


def qkv_weight_bf16(shape: LayerShape, config: int, std: float = 0.02):
    return gaussian_bf16((shape.qkv_n, shape.H), std, config, 12)


def grad_output_bf16(shape: LayerShape, config: int):
    return gaussian_bf16((shape.T, shape.H), 1.0, config, 13)
