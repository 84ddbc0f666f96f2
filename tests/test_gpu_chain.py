"""The layer at full size (4096 tokens, hidden 2048, 128 experts, top-8,
intermediate 768) as a chain: every GPU stage's output is the input of the next
oracle stage, so each kernel is checked on the values the real path feeds it.

Forward (the down path): quantize-permute, gate_up, weighted SwiGLU +
quantise, down, combine.  Backward (BF16 dgrad): down dgrad with the output
gradient gathered in its loads, SwiGLU backward, gate_up dgrad, combine.

Bars: bit-exact for the quantiser, maps, combines and the GPU's own SwiGLU
output re-quantised by the oracle; the SwiGLU values themselves bit-exact off
the float rounding midpoints (the two sides' exp may differ in the last
float64 bit); GEMMs within 2e-5 * sum |a w| on every row of sampled experts
(largest, smallest and random ones, full and partial 128-row tiles).
"""
import numpy as np
import pytest
import torch

import precision_moe_gemm_amd as pmg
import workloads as W
from oracle import combine as oc, formats as of, gemm as og, layer as ol, quantize as oq, swiglu as osw
from helpers import (BF16Experts, assert_within, bf16_dev, bf16_host, bf16_midpoint_adjacent, dev, gpu_ready,
                     host, quantize_weights_gpu_tiled, quantize_weights_oracle, sample_rows)

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_ready(), reason="needs a GPU")]


@pytest.mark.parametrize("kind", ["softmax", "zipf"])
def test_layer_forward_and_dgrad_chain(kind):
    S = W.LayerShape()
    T, H, E, k, I = S.T, S.H, S.E, S.k, S.I
    cfg = W.CFG_LAYER
    print(f"[chain] {kind}: inputs", flush=True)
    x = W.activations(T, H, config=cfg)
    ids, tw = W.make_routing(kind, T, E, k, cfg)
    wgu_bits, wd_bits = W.moe_weights_bf16(S, cfg)
    dy_bits = W.grad_output_bf16(S, cfg)
    q_gu, q_d = quantize_weights_gpu_tiled(wgu_bits), quantize_weights_gpu_tiled(wd_bits)
    tw_d = dev(tw.reshape(-1))

    print(f"[chain] {kind}: quantize-permute", flush=True)
    q = pmg.nvfp4_quantize_permute(bf16_dev(x), dev(ids), E)
    off_d, r2t_d, t2r_d = q["expert_offsets"], q["row_to_tk"], q["tk_to_row"]
    (off, r2t, t2r), a_ref = ol.quantize_permute_ref(x, ids, E)
    R = int(off[-1])
    assert np.array_equal(host(off_d), off) and np.array_equal(host(t2r_d), t2r)
    assert np.array_equal(host(r2t_d)[:R], r2t)
    for got, ref in zip((q["codes"], q["bscales"], q["rscales"]), a_ref):
        assert np.array_equal(host(got)[:R].view(np.uint8), ref.view(np.uint8))

    counts = np.diff(off)
    rows, experts = sample_rows(off, [int(np.argmax(counts)), int(np.argmin(counts))], extra=4, seed=11)
    print(f"[chain] {kind}: gate_up GEMM, experts {experts} ({rows.size} rows)", flush=True)
    gu = pmg.nvfp4_grouped_gemm(q["codes"], q["bscales"], q["rscales"], off_d, *q_gu)
    gu_h = host(gu)
    ref, bound = og.grouped_gemm_ref(*a_ref, off, *quantize_weights_oracle(wgu_bits, experts), rows=rows)
    print("  err/bound", assert_within(gu_h[rows], ref, bound, "gate_up"))

    print(f"[chain] {kind}: weighted SwiGLU + quantise on the GPU's gate_up output", flush=True)
    a2 = pmg.swiglu_quantize(gu, off_d, tw_d, r2t_d, h_out=True)
    rc, rb, rs, rh, amb = osw.swiglu_quantize_ref(gu_h[:R], osw.row_weights(tw, r2t))
    gh = host(a2[3])[:R]
    same = gh.view(np.uint32) == rh.view(np.uint32)
    assert np.all(same | amb), f"h differs off the midpoints at {np.argwhere(~(same | amb))[:5].tolist()}"
    a2_h = tuple(host(t)[:R] for t in a2[:3])
    for got, want in zip(a2_h, oq.quantize_rows_f32(gh)):      # every row, from the GPU's own h
        assert np.array_equal(got.view(np.uint8), want.view(np.uint8))
    clean = ~amb.any(axis=1)
    print(f"  midpoint-adjacent elements: {int(amb.sum())} in {int((~clean).sum())} rows", flush=True)
    for got, want in zip(a2_h, (rc, rb, rs)):                   # rows without one: the oracle's own bytes
        assert np.array_equal(got[clean].view(np.uint8), want[clean].view(np.uint8))

    print(f"[chain] {kind}: down GEMM on the GPU's quantised SwiGLU output", flush=True)
    d = pmg.nvfp4_grouped_gemm(a2[0], a2[1], a2[2], off_d, *q_d)
    d_h = host(d)
    ref, bound = og.grouped_gemm_ref(*a2_h, off, *quantize_weights_oracle(wd_bits, experts), rows=rows)
    print("  err/bound", assert_within(d_h[rows], ref, bound, "down"))

    print(f"[chain] {kind}: combine", flush=True)
    y = pmg.unpermute_combine(d, t2r_d, k)
    ry, _ = oc.unpermute_combine_ref(d_h[:R], t2r, k)
    assert np.array_equal(bf16_host(y), ry)

    print(f"[chain] {kind}: dgrad down (dY gathered in the loads)", flush=True)
    wd_dev, wgu_dev = bf16_dev(wd_bits), bf16_dev(wgu_bits)
    dh = pmg.bf16_grouped_gemm_gather(bf16_dev(dy_bits), r2t_d, k, off_d, wd_dev, pmg.W_KN)
    dh_h = host(dh)
    dy_perm = oc.permute_gather_ref(dy_bits, r2t, k)
    ref, bound = og.bf16_grouped_gemm_ref(of.bf16_to_f32(dy_perm), off, BF16Experts(wd_bits), trans_w=False,
                                          rows=rows)
    print("  err/bound", assert_within(dh_h[rows], ref, bound, "dgrad down"))

    print(f"[chain] {kind}: SwiGLU backward on the GPU's gate_up output and dH", flush=True)
    dgu = pmg.swiglu_backward(gu, dh, off_d, tw_d, r2t_d)
    dgu_h = bf16_host(dgu)[:R]
    ref_bits, d64 = osw.swiglu_backward_ref(gu_h[:R], dh_h[:R], osw.row_weights(tw, r2t))
    diff = dgu_h != ref_bits
    amb_b = bf16_midpoint_adjacent(d64)
    assert not np.any(diff & ~amb_b), f"{int((diff & ~amb_b).sum())} bf16 values differ"
    del d64, ref_bits

    print(f"[chain] {kind}: dgrad gate_up on the GPU's SwiGLU gradient", flush=True)
    dxp = pmg.bf16_grouped_gemm(dgu, off_d, wgu_dev, pmg.W_KN)
    dxp_h = host(dxp)
    ref, bound = og.bf16_grouped_gemm_ref(of.bf16_to_f32(dgu_h), off, BF16Experts(wgu_bits), trans_w=False,
                                          rows=rows)
    print("  err/bound", assert_within(dxp_h[rows], ref, bound, "dgrad gate_up"))

    print(f"[chain] {kind}: dgrad combine", flush=True)
    dx = pmg.unpermute_combine(dxp, t2r_d, k)
    rdx, _ = oc.unpermute_combine_ref(dxp_h[:R], t2r, k)
    assert np.array_equal(bf16_host(dx), rdx)
    torch.cuda.synchronize()
