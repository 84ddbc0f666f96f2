"""The gate_up GEMM with the weighted SwiGLU in its epilogue
(nvfp4_grouped_gemm_swiglu) and the FP32-row quantiser that follows it.

Contract (the SwiGLU in FP32):
  (i)  h is within 2^-20 |h64| + 2^-24 max_row |h64| of h64, the oracle's float64
       weighted SwiGLU of the same g and u;
  (ii) the NVFP4 bytes of every routed row are the oracle's quantiser applied
       to the GPU's own h.
The gate/up values the fused kernel writes for the backward are bit-identical
to the plain grouped GEMM's output, which is itself checked against the oracle
here on sampled experts; h does not depend on whether they are written.
"""
import numpy as np
import pytest
import torch

import precision_moe_gemm_amd as pmg
import workloads as W
from oracle import gemm as og, layer as ol, quantize as oq, swiglu as osw
from helpers import (assert_within, bf16_dev, dev, gpu_ready, host, quantize_weights_gpu_tiled,
                     quantize_weights_oracle, sample_rows)

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_ready(), reason="needs a GPU")]


@pytest.mark.parametrize("T,H,E,k,I,kind,weighted", [
    (4096, 2048, 128, 8, 768, "softmax", True),     # the layer's gate_up (three 256-column h tiles)
    (4096, 2048, 128, 8, 768, "zipf", True),
    (300, 256, 16, 4, 256, "uniform", False),       # one h tile, ragged experts, no router weight
    (37, 512, 8, 2, 512, "zipf", True),             # tiny experts, K = 512
    (256, 256, 1024, 8, 256, "uniform", True),      # the most experts
])
def test_fused_gate_up_swiglu(T, H, E, k, I, kind, weighted):
    print(f"[fused swiglu] T={T} H={H} E={E} k={k} I={I} {kind} weighted={weighted}", flush=True)
    x = W.activations(T, H, config=W.CFG_DOWN, tensor=7)
    ids, tw = W.make_routing(kind, T, E, k, W.CFG_DOWN)
    w_bits = W.gaussian_bf16((E, 2 * I, H), 0.02, W.CFG_DOWN, 22)
    wq = quantize_weights_gpu_tiled(w_bits)
    q = pmg.nvfp4_quantize_permute(bf16_dev(x), dev(ids), E)
    a = (q["codes"], q["bscales"], q["rscales"], q["expert_offsets"])
    tw_d = dev(tw.reshape(-1)) if weighted else None
    r2t = q["row_to_tk"] if weighted else None
    gu_plain = host(pmg.nvfp4_grouped_gemm(*a, *wq))
    h, gu = pmg.nvfp4_grouped_gemm_swiglu(*a, *wq, topk_w=tw_d, row_to_tk=r2t, want_gu=True)
    h_only, _ = pmg.nvfp4_grouped_gemm_swiglu(*a, *wq, topk_w=tw_d, row_to_tk=r2t)
    codes, bsc, rsc = pmg.nvfp4_quantize_rows_f32(h, q["expert_offsets"])
    torch.cuda.synchronize()
    off = host(q["expert_offsets"])
    R = int(off[-1])
    gu_h, h_h = host(gu)[:R], host(h)[:R]
    assert np.array_equal(gu_h.view(np.uint32), gu_plain[:R].view(np.uint32)), "gate/up differ from the plain GEMM"
    assert np.array_equal(host(h_only)[:R].view(np.uint32), h_h.view(np.uint32))
    # the gate/up values against the oracle on sampled experts
    (off_r, r2t_r, _), a_ref = ol.quantize_permute_ref(x, ids, E)
    counts = np.diff(off_r)
    rows, experts = sample_rows(off_r, [int(np.argmax(counts)), int(np.argmin(counts))], extra=2, seed=3)
    ref, bound = og.grouped_gemm_ref(*a_ref, off_r, *quantize_weights_oracle(w_bits, experts), rows=rows)
    assert_within(gu_h[rows], ref, bound, "fused gate_up")
    # (i) h against the float64 SwiGLU of the same g and u
    h64 = osw.swiglu_h64(gu_h, osw.row_weights(tw, r2t_r) if weighted else None)
    amax = np.abs(h64).max(axis=1, keepdims=True)
    tol = 2.0 ** -20 * np.abs(h64) + 2.0 ** -24 * amax
    err = np.abs(h_h.astype(np.float64) - h64)
    print(f"  h err/tol max {float((err / np.maximum(tol, 1e-300)).max()):.3g}", flush=True)
    assert np.all(err <= tol), f"h outside the tolerance at {np.argwhere(err > tol)[:5].tolist()}"
    # (ii) the quantiser's bytes from the GPU's own h
    for got, want in zip((codes, bsc, rsc), oq.quantize_rows_f32(h_h)):
        assert np.array_equal(host(got)[:R].view(np.uint8), want.view(np.uint8))
