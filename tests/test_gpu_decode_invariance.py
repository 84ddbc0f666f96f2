"""Decode-shaped batches give the same bits as the full batch.

A token's codes, scales, GEMM rows, SwiGLU-quantised rows and combined output
must not depend on how many other tokens share the call: per-token scaling
makes the quantiser row-local, and every kernel's reduction order is fixed per
row (the GEMMs' K order does not depend on the tile a row lands in).  The
whole forward path runs on 512 tokens and again on decode-sized subsets
(1 to 8 tokens, with their own routing rows), and the results are compared
bit for bit, token by token.
"""
import numpy as np
import pytest
import torch

import precision_moe_gemm_amd as pmg
import workloads as W
from helpers import bf16_dev, dev, gpu_ready, host, quantize_weights_gpu_tiled

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_ready(), reason="needs a GPU")]

T, H, E, K_TOP, I = 512, 512, 16, 4, 128


def _forward(x_bits, ids, tw, wgu, wd):
    """Routed forward: quantize-permute, gate_up, weighted SwiGLU + quantise,
    down, combine.  Returns per-(token, slot) rows of every stage and y."""
    q = pmg.nvfp4_quantize_permute(bf16_dev(x_bits), dev(ids), E)
    off, t2r, r2t = q["expert_offsets"], q["tk_to_row"], q["row_to_tk"]
    gu = pmg.nvfp4_grouped_gemm(q["codes"], q["bscales"], q["rscales"], off, *wgu)
    a2 = pmg.swiglu_quantize(gu, off, dev(tw.reshape(-1)), r2t)
    d = pmg.nvfp4_grouped_gemm(a2[0], a2[1], a2[2], off, *wd)
    y = pmg.unpermute_combine(d, t2r, K_TOP)
    torch.cuda.synchronize()
    rows = host(t2r).reshape(-1)
    pick = lambda t: host(t)[rows]
    return {"codes": pick(q["codes"]), "bscales": pick(q["bscales"]),
            "rscales": pick(q["rscales"]).view(np.uint32), "gate_up": pick(gu).view(np.uint32),
            "a2_codes": pick(a2[0]), "a2_bscales": pick(a2[1]),
            "a2_rscales": pick(a2[2]).view(np.uint32), "down": pick(d).view(np.uint32),
            "y": host(y.view(torch.int16)).view(np.uint16)}


def test_decode_sized_batches_match_the_full_batch():
    print(f"[decode invariance] T={T} H={H} E={E} k={K_TOP} I={I}", flush=True)
    x = W.activations(T, H, config=50)
    ids, tw = W.make_routing("softmax", T, E, K_TOP, 50)
    wgu = quantize_weights_gpu_tiled(W.gaussian_bf16((E, 2 * I, H), 0.02, 50, 1))
    wd = quantize_weights_gpu_tiled(W.gaussian_bf16((E, H, I), 0.02, 50, 2))
    full = _forward(x, ids, tw, wgu, wd)
    per_tok = lambda v, t0, t1: v[t0 * K_TOP:t1 * K_TOP] if v.shape[0] == T * K_TOP else v[t0:t1]
    for t0, t1 in [(0, 1), (7, 10), (100, 108), (511, 512)]:
        print(f"[decode invariance] tokens {t0}..{t1 - 1}", flush=True)
        part = _forward(np.ascontiguousarray(x[t0:t1]), np.ascontiguousarray(ids[t0:t1]),
                        np.ascontiguousarray(tw[t0:t1]), wgu, wd)
        for name in full:
            assert np.array_equal(part[name], per_tok(full[name], t0, t1)), (name, t0, t1)
