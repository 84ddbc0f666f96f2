"""Decode-shaped batches give the same bits as the full batch.

A token's codes, scales, GEMM rows, SwiGLU-quantised rows and combined output
must not depend on how many other tokens share the call: per-token scaling
makes the quantiser row-local, and every kernel's reduction order is fixed per
row (the GEMMs' K order does not depend on the tile a row lands in).  The
whole forward path runs on 512 tokens and again on decode-sized subsets
(1 to 8 tokens, with their own routing rows), and the results are compared
bit for bit, token by token.  Each decode-sized run is also compared with the
oracle, stage by stage (every GPU stage's output feeding the next oracle
stage): quantiser bytes and maps bit-exact, GEMM rows within
2e-5 * sum |a w|, the SwiGLU values off rounding midpoints and the bytes of
the GPU's own SwiGLU output re-quantised bit-exact, the combine bit-exact.
"""
import numpy as np
import pytest
import torch

import precision_moe_gemm_amd as pmg
import workloads as W
from oracle import combine as oc, gemm as og, layer as ol, quantize as oq, swiglu as osw
from helpers import (assert_within, bf16_dev, bf16_host, dev, gpu_ready, host, quantize_weights_gpu_tiled,
                     quantize_weights_oracle)

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


def _check_with_oracle(x_bits, ids, tw, wgu_bits, wd_bits, wgu, wd):
    """One decode-sized forward on the GPU, each stage against the oracle stage fed
    with the GPU's previous output."""
    q = pmg.nvfp4_quantize_permute(bf16_dev(x_bits), dev(ids), E)
    off_d = q["expert_offsets"]
    (off, r2t, t2r), a_ref = ol.quantize_permute_ref(x_bits, ids, E)
    R = int(off[-1])
    assert np.array_equal(host(off_d), off) and np.array_equal(host(q["tk_to_row"]), t2r)
    for got, ref in zip((q["codes"], q["bscales"], q["rscales"]), a_ref):
        assert np.array_equal(host(got)[:R].view(np.uint8), ref.view(np.uint8))
    gu = pmg.nvfp4_grouped_gemm(q["codes"], q["bscales"], q["rscales"], off_d, *wgu)
    gu_h = host(gu)[:R]
    ref, bound = og.grouped_gemm_ref(*a_ref, off, *quantize_weights_oracle(wgu_bits))
    assert_within(gu_h, ref, bound, "decode gate_up")
    a2 = pmg.swiglu_quantize(gu, off_d, dev(tw.reshape(-1)), q["row_to_tk"], h_out=True)
    rc, rb, rs, rh, amb = osw.swiglu_quantize_ref(gu_h, osw.row_weights(tw, r2t))
    gh = host(a2[3])[:R]
    assert np.all((gh.view(np.uint32) == rh.view(np.uint32)) | amb)
    a2_h = tuple(host(t)[:R] for t in a2[:3])
    for got, want in zip(a2_h, oq.quantize_rows_f32(gh)):
        assert np.array_equal(got.view(np.uint8), want.view(np.uint8))
    d = pmg.nvfp4_grouped_gemm(a2[0], a2[1], a2[2], off_d, *wd)
    d_h = host(d)[:R]
    ref, bound = og.grouped_gemm_ref(*a2_h, off, *quantize_weights_oracle(wd_bits))
    assert_within(d_h, ref, bound, "decode down")
    y = pmg.unpermute_combine(d, q["tk_to_row"], K_TOP)
    assert np.array_equal(bf16_host(y), oc.unpermute_combine_ref(d_h, t2r, K_TOP)[0])


def test_decode_sized_batches_match_the_full_batch():
    print(f"[decode invariance] T={T} H={H} E={E} k={K_TOP} I={I}", flush=True)
    x = W.activations(T, H, config=50)
    ids, tw = W.make_routing("softmax", T, E, K_TOP, 50)
    wgu_bits = W.gaussian_bf16((E, 2 * I, H), 0.02, 50, 1)
    wd_bits = W.gaussian_bf16((E, H, I), 0.02, 50, 2)
    wgu, wd = quantize_weights_gpu_tiled(wgu_bits), quantize_weights_gpu_tiled(wd_bits)
    full = _forward(x, ids, tw, wgu, wd)
    per_tok = lambda v, t0, t1: v[t0 * K_TOP:t1 * K_TOP] if v.shape[0] == T * K_TOP else v[t0:t1]
    for t0, t1 in [(0, 1), (7, 10), (100, 108), (511, 512)]:
        print(f"[decode invariance] tokens {t0}..{t1 - 1}", flush=True)
        part = _forward(np.ascontiguousarray(x[t0:t1]), np.ascontiguousarray(ids[t0:t1]),
                        np.ascontiguousarray(tw[t0:t1]), wgu, wd)
        for name in full:
            assert np.array_equal(part[name], per_tok(full[name], t0, t1)), (name, t0, t1)
        _check_with_oracle(np.ascontiguousarray(x[t0:t1]), np.ascontiguousarray(ids[t0:t1]),
                           np.ascontiguousarray(tw[t0:t1]), wgu_bits, wd_bits, wgu, wd)
