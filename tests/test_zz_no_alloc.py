"""The allocation-free quantize-permute (nvfp4_quantize_permute_noalloc, device
scratch inside the library) against the workspace entry point
(nvfp4_quantize_permute): identical bytes, maps and offsets, on calls in a row
whose later ones are smaller than earlier ones (the scratch keeps the last
call's contents), including the largest routing list the scratch holds.
"""
import numpy as np
import pytest
import torch

import precision_moe_gemm_amd as pmg
import workloads as W
from helpers import bf16_dev, dev

pytestmark = pytest.mark.gpu

# (T, H, E, k, routing): the headline shape, a smaller one, the largest list the
# scratch takes (one chunk table per 4096 entries, long-list plan), a tiny one
CASES = [(4096, 2048, 128, 8, "softmax"), (300, 512, 16, 4, "uniform"),
         (pmg.NOALLOC_MAX_ENTRIES // 8, 64, 128, 8, "zipf"), (5, 32, 4, 2, "uniform")]


def _outputs(T, H, E, k):
    R = T * k
    u8 = lambda *s: torch.full(s, 0xA5, dtype=torch.uint8, device="cuda")
    i32 = lambda *s: torch.full(s, -7, dtype=torch.int32, device="cuda")
    return {"codes": u8(R, H // 2), "bscales": u8(R, H // 16),
            "rscales": torch.full((R,), float("nan"), dtype=torch.float32, device="cuda"),
            "expert_offsets": i32(E + 1), "row_to_tk": i32(R), "tk_to_row": i32(R)}


def test_noalloc_matches_workspace_entry_point():
    for T, H, E, k, kind in CASES:
        print(f"[noalloc] T={T} H={H} E={E} k={k} {kind}", flush=True)
        x = bf16_dev(W.activations(T, H, config=2, tensor=40))
        ids_np, _ = W.make_routing(kind, T, E, k, 40)
        ids = dev(ids_np)
        ref = pmg.nvfp4_quantize_permute(x, ids, E)
        out = _outputs(T, H, E, k)
        torch.cuda.synchronize()
        before = torch.cuda.memory_allocated()
        pmg.nvfp4_quantize_permute_noalloc(x, ids, E, out)
        torch.cuda.synchronize()
        assert torch.cuda.memory_allocated() == before
        R = int(ref["expert_offsets"][-1].item())
        assert R == T * k
        for name in ("expert_offsets", "tk_to_row"):
            assert torch.equal(out[name], ref[name]), name
        for name in ("row_to_tk", "codes", "bscales"):
            assert torch.equal(out[name][:R], ref[name][:R]), name
        assert torch.equal(out["rscales"][:R].view(torch.int32), ref["rscales"][:R].view(torch.int32))


def test_noalloc_refuses_more_than_the_scratch():
    T, k = pmg.NOALLOC_MAX_ENTRIES // 8 + 1, 8
    x = torch.zeros(T, 16, dtype=torch.bfloat16, device="cuda")
    ids = torch.zeros(T, k, dtype=torch.int32, device="cuda")
    with pytest.raises(pmg.NVFP4Error, match="scratch"):
        pmg.nvfp4_quantize_permute_noalloc(x, ids, 8, _outputs(T, 16, 8, k))
