"""A whole layer step captured in a HIP graph replays to the eager results.

Every entry point enqueues kernels only (no allocation, copy or fill), so the
step's calls can be captured as they are.  The graph is replayed three times;
between replays eager work overwrites every output, and each replay's outputs
must equal the eager step's bit for bit.
"""
import numpy as np
import pytest
import torch

import precision_moe_gemm_amd as pmg
import workloads as W
from helpers import bf16_dev, dev, gpu_ready

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_ready(), reason="needs a GPU")]

T, H, E, K_TOP, I = 256, 256, 8, 4, 256


def _tiled(w2d, n):
    c, b, s = pmg.nvfp4_quantize_rows_tiled(w2d, n)
    return c, b, s.view(-1, n)


def test_layer_step_graph_replays_match_eager():
    print(f"[graph] layer step T={T} H={H} E={E} k={K_TOP} I={I}", flush=True)
    R = T * K_TOP
    x = bf16_dev(W.activations(T, H, config=7, tensor=1))
    ids_np, tw_np = W.make_routing("softmax", T, E, K_TOP, 7)
    ids, tw = dev(ids_np), dev(tw_np.reshape(-1))
    wgu = bf16_dev(W.gaussian_bf16((E, 2 * I, H), 0.02, 7, 2))
    wd = bf16_dev(W.gaussian_bf16((E, H, I), 0.02, 7, 3))
    dy = bf16_dev(W.gaussian_bf16((T, H), 1.0, 7, 4))
    q_gu = _tiled(wgu.view(E * 2 * I, H), 2 * I)
    q_d = _tiled(wd.view(E * H, I), H)
    ws = torch.empty(pmg.permute_workspace_size(T, K_TOP, E), dtype=torch.uint8, device="cuda")
    u8, f32, i32, b16 = torch.uint8, torch.float32, torch.int32, torch.bfloat16
    emp = lambda shape, dt: torch.empty(shape, dtype=dt, device="cuda")
    perm = {"codes": emp((R, H // 2), u8), "bscales": emp((R, H // 16), u8), "rscales": emp((R,), f32),
            "expert_offsets": emp((E + 1,), i32), "row_to_tk": emp((R,), i32), "tk_to_row": emp((R,), i32)}
    gu, dn, dh, dxp = emp((R, 2 * I), f32), emp((R, H), f32), emp((R, I), f32), emp((R, H), f32)
    a2 = {"codes": emp((R, I // 2), u8), "bscales": emp((R, I // 16), u8), "rscales": emp((R,), f32)}
    y, dx, dgu = emp((T, H), b16), emp((T, H), b16), emp((R, 2 * I), b16)
    h, gu2 = emp((R, I), f32), emp((R, 2 * I), f32)
    a3 = {"codes": emp((R, I // 2), u8), "bscales": emp((R, I // 16), u8), "rscales": emp((R,), f32)}
    fws = emp((pmg.workspace_size(pmg.OP_GROUPED_GEMM_SWIGLU, R_max=R),), u8)
    off = perm["expert_offsets"]

    def step():
        pmg.nvfp4_quantize_permute(x, ids, E, workspace=ws, out=perm)
        pmg.nvfp4_grouped_gemm(perm["codes"], perm["bscales"], perm["rscales"], off, *q_gu, c=gu)
        pmg.swiglu_quantize(gu, off, tw, perm["row_to_tk"], out=a2)
        pmg.nvfp4_grouped_gemm(a2["codes"], a2["bscales"], a2["rscales"], off, *q_d, c=dn)
        pmg.unpermute_combine(dn, perm["tk_to_row"], K_TOP, y=y)
        pmg.bf16_grouped_gemm_gather(dy, perm["row_to_tk"], K_TOP, off, wd, pmg.W_KN, c=dh)
        pmg.swiglu_backward(gu, dh, off, tw, perm["row_to_tk"], dgu=dgu)
        pmg.bf16_grouped_gemm(dgu, off, wgu, pmg.W_KN, c=dxp)
        pmg.unpermute_combine(dxp, perm["tk_to_row"], K_TOP, y=dx)
        # the fused gate_up + SwiGLU path (router-weight gather + GEMM) and its quantiser
        pmg.nvfp4_grouped_gemm_swiglu(perm["codes"], perm["bscales"], perm["rscales"], off, *q_gu, topk_w=tw,
                                      row_to_tk=perm["row_to_tk"], h=h, gu=gu2, workspace=fws)
        pmg.nvfp4_quantize_rows_f32(h, off, a3["codes"], a3["bscales"], a3["rscales"])

    outs = {"y": y, "dx": dx, "gu": gu, "dn": dn, "dh": dh, "dgu": dgu, "dxp": dxp, "h": h, "gu2": gu2,
            **{f"a3.{k}": v for k, v in a3.items()},
            **{f"perm.{k}": v for k, v in perm.items()}, **{f"a2.{k}": v for k, v in a2.items()}}
    step()
    torch.cuda.synchronize()
    ref = {k: v.clone() for k, v in outs.items()}

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep in range(3):
        for v in outs.values():            # eager work between replays: clobber every output
            v.view(torch.uint8).fill_(0xA5 + rep)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, v in outs.items():
            assert torch.equal(v.view(torch.uint8), ref[k].view(torch.uint8)), f"replay {rep}: {k}"
    print("  3 replays equal the eager step", flush=True)
