"""GPU parity: grouped NVFP4 GEMM against the exact-dequantisation FP64 oracle.

Bar: |C_gpu - C_ref| <= 2e-5 * sum_k |a_k w_k| for every compared element.
Small cases compare every element; the full 32768 x 1536 x 2048 gate_up and
the QKV / down shapes compare all rows of a few experts plus random rows (the
oracle computes rows one expert at a time).
"""
import numpy as np
import pytest
import torch

import precision_moe_gemm_amd as pmg
import workloads as W
from oracle import gemm as og, layer as ol, permute as op, quantize as oq
from helpers import (assert_within, bf16_dev, dev, host, gpu_ready, quantize_weights_gpu,
                     quantize_weights_gpu_tiled, quantize_weights_oracle, sample_rows)

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_ready(), reason="needs a GPU")]


def test_tiny_single_expert_gemm():
    """A [64x256] x W [128x256]^T, single expert (C = A W^T)."""
    print("[gemm] tiny 64x128x256", flush=True)
    a_bits = W.gaussian_bf16((64, 256), 1.0, W.CFG_TINY, 0)
    w_bits = W.gaussian_bf16((1, 128, 256), 1.0, W.CFG_TINY, 1)
    a = pmg.nvfp4_quantize_rows(bf16_dev(a_bits))
    w = quantize_weights_gpu(w_bits)
    off = np.array([0, 64], np.int32)
    c = pmg.nvfp4_grouped_gemm(*a, dev(off), *w)
    torch.cuda.synchronize()
    ref, bound = og.grouped_gemm_ref(*oq.quantize_rows_bf16(a_bits), off, *quantize_weights_oracle(w_bits))
    print("  err/bound", assert_within(host(c), ref, bound, "tiny"))


def _routed_case(T, H, E, k, N, kind, seed):
    x = W.activations(T, H, config=seed)
    ids, _ = W.make_routing(kind, T, E, k, seed)
    w_bits = W.gaussian_bf16((E, N, H), 0.02, seed, 20)
    res = pmg.nvfp4_quantize_permute(bf16_dev(x), dev(ids), E)
    a = (res["codes"], res["bscales"], res["rscales"], res["expert_offsets"])
    c = host(pmg.nvfp4_grouped_gemm(*a, *quantize_weights_gpu(w_bits)))
    # the K-tiled weight layout is the same computation on moved bytes
    (off, r2t, t2r), a_ref = ol.quantize_permute_ref(x, ids, E)
    R = int(off[-1])
    if H % 64 == 0:
        wt = quantize_weights_gpu_tiled(w_bits)
        ct = host(pmg.nvfp4_grouped_gemm(*a, *wt))
        assert np.array_equal(ct[:R], c[:R]), "K-tiled weights change the result"
        # BF16 output: each FP32 result rounded to nearest even; rows past the routed ones untouched
        cb = torch.full((T * k, N), -1, dtype=torch.int16, device="cuda").view(torch.bfloat16)
        pmg.nvfp4_grouped_gemm(*a, *wt, c=cb)
        cb_h = host(cb.view(torch.int16)).view(np.uint16)
        assert np.array_equal(cb_h[:R], W.f32_to_bf16_bits(c[:R])), "BF16 output is not the rounded FP32 output"
        assert np.all(cb_h[R:] == 0xFFFF)
    return c, off, a_ref, w_bits


@pytest.mark.parametrize("T,H,E,k,N,kind", [
    (512, 256, 8, 4, 256, "uniform"),      # several m/n tiles per expert, ragged tails
    (300, 512, 16, 2, 144, "zipf"),        # N not a multiple of the 128-column tile
    (64, 128, 32, 8, 16, "uniform"),       # smallest K step and N; many tiny experts
    (33, 384, 128, 8, 64, "zipf"),         # empty experts, 1-row experts
    (100, 64, 8, 4, 96, "uniform"),        # K = 64: one K-step per tile
    (2000, 64, 64, 8, 512, "zipf"),        # one K-step per tile, several tiles per workgroup
    (256, 128, 1024, 8, 64, "uniform"),    # the most experts: the prologue's tables over 1024 experts
])
def test_grouped_gemm_small_all_elements(T, H, E, k, N, kind):
    print(f"[gemm] T={T} H={H} E={E} k={k} N={N} {kind}", flush=True)
    c, off, a_ref, w_bits = _routed_case(T, H, E, k, N, kind, seed=31)
    ref, bound = og.grouped_gemm_ref(*a_ref, off, *quantize_weights_oracle(w_bits))
    R = int(off[-1])
    print("  err/bound", assert_within(c[:R], ref, bound, "small"))


@pytest.mark.parametrize("kind", ["uniform", "zipf"])
def test_gate_up_full_size_sampled(kind):
    """32768 routed rows (top-8 of 4096 tokens, 128 experts), K=2048, N=1536."""
    print(f"[gemm] gate_up full {kind}", flush=True)
    c, off, a_ref, w_bits = _routed_case(4096, 2048, 128, 8, 1536, kind, seed=W.CFG_GATEUP)
    counts = np.diff(off)
    rows, experts = sample_rows(off, [int(np.argmax(counts)), int(np.argmin(counts)), 77], extra=5, seed=1)
    ref, bound = og.grouped_gemm_ref(*a_ref, off, *quantize_weights_oracle(w_bits, experts), rows=rows)
    print("  rows", rows.size, "err/bound", assert_within(c[rows], ref, bound, f"gate_up {kind}"))
    assert np.isfinite(c[: int(off[-1])]).all()


def test_down_shape_sampled():
    """K=768, N=2048 over 128 experts (the down projection's shape), 4096 tokens:
    about 256 rows per expert, so the sampled experts hold full 128-row tiles."""
    print("[gemm] down shape", flush=True)
    T, E, k, I, H = 4096, 128, 8, 768, 2048
    x = W.activations(T, I, config=W.CFG_DOWN)
    ids, _ = W.make_routing("softmax", T, E, k, W.CFG_DOWN)
    w_bits = W.gaussian_bf16((E, H, I), 0.02, W.CFG_DOWN, 21)
    res = pmg.nvfp4_quantize_permute(bf16_dev(x), dev(ids), E)
    w = quantize_weights_gpu(w_bits)
    c = host(pmg.nvfp4_grouped_gemm(res["codes"], res["bscales"], res["rscales"], res["expert_offsets"], *w))
    (off, _, _), a_ref = ol.quantize_permute_ref(x, ids, E)
    counts = np.diff(off)
    assert counts.max() >= 256
    rows, experts = sample_rows(off, [0, 5, 127, int(np.argmax(counts))], extra=5, seed=2)
    ref, bound = og.grouped_gemm_ref(*a_ref, off, *quantize_weights_oracle(w_bits, experts), rows=rows)
    print("  err/bound", assert_within(c[rows], ref, bound, "down"))


def test_dense_qkv_sampled():
    """Dense W4A4 QKV: M=4096, K=2048, N=5120 as a one-group GEMM."""
    print("[gemm] qkv dense", flush=True)
    x = W.activations(4096, 2048, config=W.CFG_LAYER)
    w_bits = W.gaussian_bf16((1, 5120, 2048), 0.02, W.CFG_LAYER, 12)
    a = pmg.nvfp4_quantize_rows(bf16_dev(x))
    w = quantize_weights_gpu(w_bits)
    off = np.array([0, 4096], np.int32)
    c = host(pmg.nvfp4_grouped_gemm(*a, dev(off), *w))
    rows = np.unique(np.concatenate([np.arange(0, 130), np.arange(3990, 4096),
                                     np.random.default_rng(3).integers(0, 4096, 40)]))
    ref, bound = og.grouped_gemm_ref(*oq.quantize_rows_bf16(x), off, *quantize_weights_oracle(w_bits), rows=rows)
    print("  err/bound", assert_within(c[rows], ref, bound, "qkv"))


def test_rows_are_batch_invariant():
    """A token's GEMM row does not depend on how many other rows the expert has."""
    print("[gemm] batch invariance", flush=True)
    T, H, N = 300, 512, 256
    x = W.activations(T, H, config=40)
    w_bits = W.gaussian_bf16((1, N, H), 0.02, 40, 1)
    w = quantize_weights_gpu(w_bits)
    a = pmg.nvfp4_quantize_rows(bf16_dev(x))
    full = host(pmg.nvfp4_grouped_gemm(*a, dev(np.array([0, T], np.int32)), *w))
    for t0, t1 in [(0, 1), (5, 9), (130, 300)]:
        sub = tuple(v[t0:t1].clone() for v in a)          # fresh, aligned allocations
        part = host(pmg.nvfp4_grouped_gemm(*sub, dev(np.array([0, t1 - t0], np.int32)), *w))
        assert np.array_equal(part, full[t0:t1])


def _oracle_rows(a_bits, off, w_bits, rows):
    """oracle C rows (with their bounds) of row-quantised activations a_bits"""
    a_ref = oq.quantize_rows_bf16(a_bits)
    return og.grouped_gemm_ref(*a_ref, off, *quantize_weights_oracle(w_bits), rows=rows)


def test_quarter_tiles_dense():
    """A last round that would keep at most a quarter of a range's workgroups
    busy is split into 128-column quarter tiles.  Dense 4096 x 5120 (320 tiles
    on 256 workgroups: the last 8 of every 40-tile range become 32 quarters).
    The quarters must give the bits of whole tiles (two half-height launches,
    whose single round has no quarters) and the oracle's values on rows of
    quartered and whole m-tiles."""
    print("[gemm] quarter tiles: dense 4096x5120, K 256", flush=True)
    M, K, N = 4096, 256, 5120
    x = W.activations(M, K, config=44)
    w_bits = W.gaussian_bf16((1, N, K), 0.02, 44, 1)
    a = pmg.nvfp4_quantize_rows(bf16_dev(x))
    w = quantize_weights_gpu(w_bits)
    full = host(pmg.nvfp4_grouped_gemm(*a, dev(np.array([0, M], np.int32)), *w))
    for lo, hi in [(0, 2048), (2048, 4096)]:
        sub = tuple(v[lo:hi].clone() for v in a)
        part = host(pmg.nvfp4_grouped_gemm(*sub, dev(np.array([0, hi - lo], np.int32)), *w))
        assert np.array_equal(part.view(np.int32), full[lo:hi].view(np.int32)), f"rows {lo}..{hi}"
    # m-tile 3 (rows 384..511) has quartered columns 1024.., m-tile 0 none
    rows = np.unique(np.concatenate([np.arange(0, 40), np.arange(384, 512), np.arange(4060, 4096)]))
    ref, bound = _oracle_rows(x, np.array([0, M], np.int64), w_bits, rows)
    print("  err/bound", assert_within(full[rows], ref, bound, "quarters dense"))


def test_quarter_tiles_dense_ragged():
    """Quarter tiles with rows missing: dense 4000 x 5120, K 128, K-tiled weights
    (m-tile 31 holds 32 rows, so in its quarters one wavefront row half has a
    single 32-row fragment and the other none).  Bit-identical to two half-height
    launches without quarters; every row of m-tiles 3 and 31 against the oracle."""
    print("[gemm] quarter tiles: dense 4000x5120, K 128, K-tiled", flush=True)
    M, K, N = 4000, 128, 5120
    x = W.activations(M, K, config=45)
    w_bits = W.gaussian_bf16((1, N, K), 0.02, 45, 1)
    a = pmg.nvfp4_quantize_rows(bf16_dev(x))
    w = quantize_weights_gpu_tiled(w_bits)
    full = host(pmg.nvfp4_grouped_gemm(*a, dev(np.array([0, M], np.int32)), *w))
    for lo, hi in [(0, 2000), (2000, 4000)]:
        sub = tuple(v[lo:hi].clone() for v in a)
        part = host(pmg.nvfp4_grouped_gemm(*sub, dev(np.array([0, hi - lo], np.int32)), *w))
        assert np.array_equal(part.view(np.int32), full[lo:hi].view(np.int32)), f"rows {lo}..{hi}"
    rows = np.concatenate([np.arange(384, 512), np.arange(3968, 4000)])
    ref, bound = _oracle_rows(x, np.array([0, M], np.int64), w_bits, rows)
    print("  err/bound", assert_within(full[rows], ref, bound, "quarters ragged"))


def test_repeated_calls_are_identical():
    """Back-to-back calls (ragged experts, more tiles than workgroups) give
    bit-identical results."""
    print("[gemm] repeated calls", flush=True)
    T, H, E, k, N = 2048, 512, 16, 4, 768
    ids = W.make_routing("zipf", T, E, k, 41)[0]
    x = W.activations(T, H, config=41)
    res = pmg.nvfp4_quantize_permute(bf16_dev(x), dev(ids), E)
    w = quantize_weights_gpu(W.gaussian_bf16((E, N, H), 0.02, 41, 1))
    outs = [host(pmg.nvfp4_grouped_gemm(res["codes"], res["bscales"], res["rscales"],
                                        res["expert_offsets"], *w)) for _ in range(3)]
    R = int(host(res["expert_offsets"])[-1])
    for o in outs[1:]:
        assert np.array_equal(o[:R], outs[0][:R])


def test_binding_refuses_short_buffers():
    """The C-ABI sees pointers only: the binding refuses an output (or a known
    input) smaller than what the library would write (read), before any launch."""
    print("[binding] short buffers", flush=True)
    x = W.activations(64, 256, config=3, tensor=1)
    a = pmg.nvfp4_quantize_rows(bf16_dev(x))
    w = quantize_weights_gpu(W.gaussian_bf16((1, 128, 256), 1.0, 3, 2))
    off = dev(np.array([0, 64], np.int32))
    with pytest.raises(ValueError, match="needs"):
        pmg.nvfp4_grouped_gemm(*a, off, *w, c=torch.empty(64 * 127, dtype=torch.float32, device="cuda"))
    with pytest.raises(ValueError, match="needs"):
        pmg.nvfp4_quantize_rows(bf16_dev(x), codes=torch.empty(10, dtype=torch.uint8, device="cuda"))
    with pytest.raises(ValueError, match="needs"):
        pmg.bf16_transpose(bf16_dev(x.reshape(1, 64, 256)), out=torch.empty(8, dtype=torch.bfloat16, device="cuda"))
    # row-major weight block scales shorter than E * N * K/16
    with pytest.raises(ValueError, match="layout"):
        pmg.nvfp4_grouped_gemm(*a, off, w[0], w[1][:, :64], w[2])
    # combine: d with fewer than T * k rows; tk_to_row not a multiple of k
    t2r = dev(np.arange(16, dtype=np.int32))
    with pytest.raises(ValueError, match="needs"):
        pmg.unpermute_combine(torch.empty(15, 64, dtype=torch.float32, device="cuda"), t2r, 4)
    with pytest.raises(ValueError, match="T \\* k"):
        pmg.unpermute_combine(torch.empty(16, 64, dtype=torch.float32, device="cuda"), t2r, 3)
    # SwiGLU passes: router weights for fewer than R_cap entries
    gu = torch.zeros(16, 64, dtype=torch.float32, device="cuda")
    off16 = dev(np.array([0, 16], np.int32))
    r2t = dev(np.arange(16, dtype=np.int32))
    short_w = torch.ones(15, dtype=torch.float32, device="cuda")
    with pytest.raises(ValueError, match="needs"):
        pmg.swiglu_quantize(gu, off16, short_w, r2t)
    with pytest.raises(ValueError, match="needs"):
        pmg.swiglu_backward(gu, torch.zeros(16, 32, dtype=torch.float32, device="cuda"), off16, short_w, r2t)
    torch.cuda.synchronize()


def test_more_m_tiles_than_the_lds_table():
    """Over 8192 m-tiles of 128 rows: each tile's expert then comes from a binary
    search over the experts' first m-tiles instead of the prologue's LDS table.
    Rows are batch-invariant, so the result must equal, bit for bit, separate
    launches per expert (each within the table's reach), and the oracle on
    sampled rows.  Activations are random valid NVFP4 bytes made on the device."""
    print("[gemm] > 8192 m-tiles (search path)", flush=True)
    K, N = 64, 16
    sizes = [400_000, 1, 649_215]                       # 3125 + 1 + 5072 = 8198 m-tiles
    R = sum(sizes)
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    g = torch.Generator(device="cuda").manual_seed(5)
    codes = torch.randint(0, 256, (R, K // 2), dtype=torch.uint8, device="cuda", generator=g)
    bsc = torch.randint(0x28, 0x48, (R, K // 16), dtype=torch.uint8, device="cuda", generator=g)
    rsc = torch.rand(R, device="cuda", generator=g) + 0.5
    w_bits = W.gaussian_bf16((3, N, K), 0.02, 43, 1)
    w = quantize_weights_gpu(w_bits)
    full = pmg.nvfp4_grouped_gemm(codes, bsc, rsc, dev(off), *w)
    for e in range(3):
        lo, hi = int(off[e]), int(off[e + 1])
        part = pmg.nvfp4_grouped_gemm(codes[lo:hi].clone(), bsc[lo:hi].clone(), rsc[lo:hi].clone(),
                                      dev(np.array([0, hi - lo], np.int32)), *(t[e:e + 1].clone() for t in w))
        assert torch.equal(part.view(torch.int32), full[lo:hi].view(torch.int32)), f"expert {e}"
    rows = np.unique(np.concatenate([np.arange(0, 200), np.arange(399_990, 400_010),
                                     np.arange(R - 300, R), np.random.default_rng(4).integers(0, R, 200)]))
    a_h = (host(codes[rows]), host(bsc[rows]), host(rsc[rows]))
    e_of = np.searchsorted(off, rows, side="right") - 1
    sub_off = np.searchsorted(e_of, np.arange(4)).astype(np.int64)
    ref, bound = og.grouped_gemm_ref(*a_h, sub_off, *quantize_weights_oracle(w_bits))
    print("  err/bound", assert_within(host(full)[rows], ref, bound, "search path"))
