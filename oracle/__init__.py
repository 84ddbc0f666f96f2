"""CPU oracle for the NVFP4 W4A4 MoE hot path.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The product path
(``precision_moe_gemm_amd`` and its HIP library) never imports, links or calls
it, and the two share no code: the only common module is ``workloads`` (seeded
input synthesis, which holds none of the method's arithmetic).

Sources.  The method is described in three web pages about miniTE:
  * "miniTE accélère le RL en NVFP4 sur B300 : 1,39× par rapport à BF16 sur
    Qwen3-30B-A3B" (news.hamidun.com), §Diagnostic, alignement et noyaux rapides
    and §Paramètres clés: native NVFP4 W4A4, optimised NVFP4 kernels, scaling
    scheme and grouped GEMMs for MoE;
  * the blog post on the miniTE technical report (yuxiaoba.github.io,
    "miniTE NVFP4"), §Follow the numerical execution path: per-token scaling,
    comparison after aligning token and expert identities; §Two complementary
    interventions: contiguous buffers with device-side metadata, amax taken
    during permutation or weighted SwiGLU, scale-layout conversion fused with
    quantisation, independent forward/backward precision;
  * "Hugging Face Releases miniTE Framework" (zicq.com), §Technical Mechanism
    Analysis: W4A4 GEMM.
The pages give no formulas.  The bit format is the public NVFP4 definition
(E2M1 element codes on the grid {0, 0.5, 1, 1.5, 2, 3, 4, 6}, one E4M3 scale per
16 elements, an FP32 second-level scale, here one per token / weight row).  Each
module states the reading it takes where the pages are silent.

Modules:
  formats   - bf16 / E4M3 / E2M1 codecs (closed forms)
  quantize  - NVFP4 quantisation of rows with a per-row FP32 scale
  permute   - stable expert-major permutation of routed (token, slot) pairs
  gemm      - grouped NVFP4 GEMM by exact dequantisation, FP64 accumulation,
              and a dense bf16 GEMM in FP64
  swiglu    - weighted SwiGLU + NVFP4 quantisation, and its backward
  combine   - un-permutation with top-k combine, and the gather for dgrad
  layer     - the chained MoE layer forward and BF16 dgrad backward
  wgrad     - the expert weight gradient in NVFP4, quantised along tokens
"""
from . import formats, quantize, permute, gemm, swiglu, combine, layer, wgrad  # noqa: F401
