"""Benchmark of the NVFP4 W4A4 MoE hot path on one MI355X.

One step = one pass of the whole path over a Qwen3-30B-A3B-shaped layer at
4096 tokens (hidden 2048, 128 experts, top-8, expert intermediate 768):
  dense W4A4 QKV (quantise rows, one-group GEMM N=5120)
  -> MoE forward: route + permute + quantise, gate_up grouped GEMM (N=1536),
     weighted SwiGLU + quantise, down grouped GEMM (N=2048), combine
  -> BF16 dgrad: gather dY, grouped GEMM with W_d, SwiGLU backward, grouped
     GEMM with W_gu, combine.
Inputs (activations with 1% x20 outliers, softmax top-8 routing of N(0,1)
logits, N(0, 0.02) weights, N(0,1) dY) are synthetic and seeded, resident in
HBM before timing; weights are quantised to NVFP4 once before timing.

Prints one JSON line.  `value` is the W4A4 grouped-GEMM throughput (gate_up +
down FLOPs over their device time, HIP events on the launch stream); the
quantize-permute GB/s, every op's time and roofline fraction, the dominant
kernel's roofline object and the CPU oracle's throughput are in the same line.
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0
PEAK_F16_TFLOPS = 2500.0     # MI355X dense FP16/BF16 MFMA


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    # the GPU clock needs some tens of ms of sustained load to settle: warm up for ~40 ms
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--routing", default="softmax", choices=["softmax", "uniform", "zipf"])
    p.add_argument("--single-routing", action="store_true",
                   help="time the headline routing only (skip the other two routings' steps)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-comparisons", action="store_true",
                   help="skip the BF16 forward and NVFP4 input-gradient timings after the timed steps")
    p.add_argument("--cpu-seconds", type=float, default=15.0, help="bound on the oracle sample's CPU time")
    p.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                   help="only copy MIB MiB device to device 4 times (calibrates the HBM byte counters)")
    return p.parse_args()


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gate_up_gemm_hbm_traffic.md")
GEMM_SOURCE = os.path.join(ROOT, "precision_moe_gemm_amd", "csrc", "gemm_nvfp4.hip")


def measured_traffic():
    """HBM bytes per gate_up launch from the committed counter summary, if it was
    taken on the kernel source as it is now (else None)."""
    import hashlib
    try:
        text = open(TRAFFIC_FILE).read()
        src = hashlib.sha256(open(GEMM_SOURCE, "rb").read()).hexdigest()
    except OSError:
        return None
    for line in text.splitlines():
        if line.startswith("traffic:"):
            kv = dict(item.split("=", 1) for item in line[len("traffic:"):].split())
            if kv.get("gemm_source_sha256") == src:
                return int(kv["fetch_bytes"]) + int(kv["write_bytes"])
    return None


def copy_probe(mib: int):
    import torch
    n = mib * 1024 * 1024 // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(4):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_per_copy": n * 4}), flush=True)


def main():
    args = parse()
    if args.copy_probe:
        copy_probe(args.copy_probe)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    import precision_moe_gemm_amd as pmg
    import workloads as W

    if not os.path.exists(pmg.library_path()):
        from precision_moe_gemm_amd import build
        build.build_library()
    pmg.load_library()
    dev = torch.device("cuda:0")
    S = W.LayerShape()
    T, H, E, k, I, R = S.T, S.H, S.E, S.k, S.I, S.R
    cfg = W.CFG_LAYER

    def bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)

    # ---------------- inputs (host synthesis, then resident on the device)
    t0 = time.time()
    x_bits = W.activations(T, H, config=cfg)
    ids_np, tw_np = W.make_routing(args.routing, T, E, k, cfg)
    wgu_bits, wd_bits = W.moe_weights_bf16(S, cfg)
    wqkv_bits = W.qkv_weight_bf16(S, cfg)
    dy_bits = W.grad_output_bf16(S, cfg)
    x, dy = bf16(x_bits), bf16(dy_bits)
    ids = torch.from_numpy(ids_np).to(dev)
    tw = torch.from_numpy(np.ascontiguousarray(tw_np.reshape(-1))).to(dev)
    wgu, wd, wqkv = bf16(wgu_bits), bf16(wd_bits), bf16(wqkv_bits)
    # NVFP4 weights, quantised once (per output row FP32 scale) straight into
    # the K-tiled layout the grouped GEMM reads one contiguous block per K-step
    def tiled(w2d, n):
        c_, b_, s_ = pmg.nvfp4_quantize_rows_tiled(w2d, n)
        return c_, b_, s_.view(-1, n)
    q_gu = tiled(wgu.view(E * 2 * I, H), 2 * I)
    q_d = tiled(wd.view(E * H, I), H)
    q_qkv = tiled(wqkv, S.qkv_n)
    qkv_off = torch.tensor([0, T], dtype=torch.int32, device=dev)
    # outputs / intermediates
    ws = torch.empty(pmg.permute_workspace_size(T, k, E), dtype=torch.uint8, device=dev)
    a_qkv = {"c": torch.empty(T, H // 2, dtype=torch.uint8, device=dev),
             "b": torch.empty(T, H // 16, dtype=torch.uint8, device=dev),
             "s": torch.empty(T, dtype=torch.float32, device=dev)}
    qkv = torch.empty(T, S.qkv_n, dtype=torch.float32, device=dev)
    perm = {"codes": torch.empty(R, H // 2, dtype=torch.uint8, device=dev),
            "bscales": torch.empty(R, H // 16, dtype=torch.uint8, device=dev),
            "rscales": torch.empty(R, dtype=torch.float32, device=dev),
            "expert_offsets": torch.empty(E + 1, dtype=torch.int32, device=dev),
            "row_to_tk": torch.empty(R, dtype=torch.int32, device=dev),
            "tk_to_row": torch.empty(R, dtype=torch.int32, device=dev)}
    gu = torch.empty(R, 2 * I, dtype=torch.float32, device=dev)
    a2 = {"codes": torch.empty(R, I // 2, dtype=torch.uint8, device=dev),
          "bscales": torch.empty(R, I // 16, dtype=torch.uint8, device=dev),
          "rscales": torch.empty(R, dtype=torch.float32, device=dev)}
    dn = torch.empty(R, H, dtype=torch.float32, device=dev)
    y = torch.empty(T, H, dtype=torch.bfloat16, device=dev)
    dh = torch.empty(R, I, dtype=torch.float32, device=dev)
    dgu = torch.empty(R, 2 * I, dtype=torch.bfloat16, device=dev)
    dx_perm = torch.empty(R, H, dtype=torch.float32, device=dev)
    dx = torch.empty(T, H, dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()
    setup_s = time.time() - t0

    off = perm["expert_offsets"]
    r2t = perm["row_to_tk"]
    hbuf = torch.empty(R, I, dtype=torch.float32, device=dev)
    fws = torch.empty(pmg.workspace_size(pmg.OP_GROUPED_GEMM_SWIGLU, R_max=R), dtype=torch.uint8, device=dev)
    a_perm = (perm["codes"], perm["bscales"], perm["rscales"], off)
    mid_plain = [
        ("gate_up_gemm", lambda: pmg.nvfp4_grouped_gemm(*a_perm, *q_gu, c=gu)),
        ("swiglu_quantize", lambda: pmg.swiglu_quantize(gu, off, tw, r2t, out=a2)),
    ]
    # the weighted SwiGLU (FP32) in the gate_up GEMM's epilogue; gate/up kept for the backward
    mid_fused = [
        ("gate_up_gemm_swiglu", lambda: pmg.nvfp4_grouped_gemm_swiglu(*a_perm, *q_gu, topk_w=tw, row_to_tk=r2t,
                                                                      h=hbuf, gu=gu, workspace=fws)),
        ("quantize_h", lambda: pmg.nvfp4_quantize_rows_f32(hbuf, off, a2["codes"], a2["bscales"], a2["rscales"])),
    ]
    ops = [
        ("qkv_quantize", lambda: pmg.nvfp4_quantize_rows(x, a_qkv["c"], a_qkv["b"], a_qkv["s"])),
        ("qkv_gemm", lambda: pmg.nvfp4_grouped_gemm(a_qkv["c"], a_qkv["b"], a_qkv["s"], qkv_off, *q_qkv, c=qkv)),
        ("quantize_permute", lambda: pmg.nvfp4_quantize_permute(x, ids, E, workspace=ws, out=perm)),
        *mid_plain,
        ("down_gemm", lambda: pmg.nvfp4_grouped_gemm(a2["codes"], a2["bscales"], a2["rscales"], off, *q_d, c=dn)),
        ("combine", lambda: pmg.unpermute_combine(dn, perm["tk_to_row"], k, y=y)),
        # the output gradient's rows are gathered into expert order inside the GEMM's loads
        ("dgrad_down_gemm", lambda: pmg.bf16_grouped_gemm_gather(dy, r2t, k, off, wd, pmg.W_KN, c=dh)),
        ("swiglu_backward", lambda: pmg.swiglu_backward(gu, dh, off, tw, r2t, dgu=dgu)),
        ("dgrad_gate_up_gemm", lambda: pmg.bf16_grouped_gemm(dgu, off, wgu, pmg.W_KN, c=dx_perm)),
        ("dgrad_combine", lambda: pmg.unpermute_combine(dx_perm, perm["tk_to_row"], k, y=dx)),
    ]
    ops_fused = ops[:3] + mid_fused + ops[5:]
    stream = torch.cuda.current_stream()

    def step(events=None, ops=ops):
        for i, (_, fn) in enumerate(ops):
            if events is not None:
                events[i][0].record(stream)
            fn()
            if events is not None:
                events[i][1].record(stream)

    def set_routing(kind):
        ids_np_, tw_np_ = (ids_np, tw_np) if kind == args.routing else W.make_routing(kind, T, E, k, cfg)
        ids.copy_(torch.from_numpy(ids_np_))
        tw.copy_(torch.from_numpy(tw_np_.reshape(-1)))
        torch.cuda.synchronize()

    def timed_steps(warmup, ops_=ops):
        """warmup untimed steps, then --steps timed ones with per-op HIP events on the
        launch stream; returns (ms per step, {op: ms})"""
        for _ in range(warmup):
            step(None, ops_)
        evs = [[[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)]
                for _ in range(len(ops_))] for _ in range(args.steps)]
        start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record(stream)
        for s_ in range(args.steps):
            step(evs[s_], ops_)
        stop.record(stream)
        torch.cuda.synchronize()
        op_ms_ = {name: float(np.mean([evs[s_][i][0].elapsed_time(evs[s_][i][1]) for s_ in range(args.steps)]))
                  for i, (name, _) in enumerate(ops_)}
        return start.elapsed_time(stop) / args.steps, op_ms_

    # timed region: K full steps of the headline routing
    ms_step, op_ms = timed_steps(args.warmup)
    # the same steps with no per-op events, as the baseline of the graph replay
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for s_ in range(args.steps):
        step()
    stop.record(stream)
    torch.cuda.synchronize()
    ms_step_plain = start.elapsed_time(stop) / args.steps
    graph = graph_steps(step, args.steps, args.warmup, T)
    graph["eager_ms_per_step_no_events"] = round(ms_step_plain, 4)

    # ---------------- algorithmic work per op (useful rows only)
    Rr = int(off[-1].item())
    gemm_flops = {
        "qkv_gemm": 2.0 * T * H * S.qkv_n,
        "gate_up_gemm": 2.0 * Rr * H * 2 * I,
        "down_gemm": 2.0 * Rr * I * H,
        "dgrad_down_gemm": 2.0 * Rr * H * I,
        "dgrad_gate_up_gemm": 2.0 * Rr * 2 * I * H,
    }
    nvfp4_row = lambda K: K // 2 + K // 16 + 4
    op_bytes = {
        "qkv_quantize": T * H * 2 + T * nvfp4_row(H),
        "quantize_permute": T * H * 2 + T * k * 4 + Rr * nvfp4_row(H) + 2 * Rr * 4 + (E + 1) * 4,
        "quantize_h": Rr * I * 4 + Rr * nvfp4_row(I),
        "swiglu_quantize": Rr * 2 * I * 4 + Rr * 4 * 2 + Rr * nvfp4_row(I),
        "combine": Rr * H * 4 + T * k * 4 + T * H * 2,
        "swiglu_backward": Rr * 2 * I * 4 + Rr * I * 4 + Rr * 8 + Rr * 2 * I * 2,
        "dgrad_combine": Rr * H * 4 + T * k * 4 + T * H * 2,
    }
    # quantize-permute with x out of the caches: a 512 MiB write between launches
    # (outside the timed events) evicts the 256 MB last-level cache, so x and
    # the routing come from HBM, as they would after the attention block
    qp_cold_us = time_cold(ops[2][1], reps=args.steps)
    op_ms_in_step = dict(op_ms)
    op_ms["quantize_permute"] = qp_cold_us * 1e-3

    def per_op_of(op_ms_):
        out = {}
        for name in op_ms_:
            us = op_ms_[name] * 1e3
            d = {"us": round(us, 2)}
            if name in gemm_flops:
                tf = gemm_flops[name] / (us * 1e-6) / 1e12
                d.update(TFLOPs=round(tf, 1), frac_f16_mfma_peak=round(tf / PEAK_F16_TFLOPS, 4))
            if name in op_bytes:
                gbs = op_bytes[name] / (us * 1e-6) / 1e9
                d.update(GBps=round(gbs, 1), frac_hbm_peak=round(gbs / PEAK_HBM_GBPS, 4))
            out[name] = d
        return out

    per_op = per_op_of(op_ms)
    per_op["quantize_permute"]["in_step_us"] = round(op_ms_in_step["quantize_permute"] * 1e3, 2)
    per_op["quantize_permute"]["how"] = ("mean over --steps launches, each after a 512 MiB cache-evicting "
                                         "write outside its events; in_step_us: inside the timed step")

    w4 = lambda om: (gemm_flops["gate_up_gemm"] + gemm_flops["down_gemm"]) / (
        (om["gate_up_gemm"] + om["down_gemm"]) * 1e-3) / 1e12
    value = w4(op_ms)
    gu_us = op_ms["gate_up_gemm"] * 1e3
    gu_tf = gemm_flops["gate_up_gemm"] / (gu_us * 1e-6) / 1e12
    roofline = {"kernel": "nvfp4 grouped GEMM gate_up (grouped_gemm_kernel<K-tiled, FP32 out>)",
                "bound": "mfma", "achieved": round(gu_tf, 2), "peak": PEAK_F16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(gu_tf / PEAK_F16_TFLOPS, 4), "traffic": measured_traffic(),
                "work_per_launch": f"{gemm_flops['gate_up_gemm']:.4e} FLOP (2 * {Rr} rows * 2048 * 1536)",
                "avg_launch_us": round(gu_us, 2)}

    result = {
        "metric": "W4A4 grouped-GEMM TFLOP/s + quantize-permute GB/s, 30B-A3B MoE layer @4096 tok",
        "value": round(value, 2), "unit": "TFLOP/s",
        "quantize_permute_GBps": per_op["quantize_permute"]["GBps"],
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f16 (NVFP4 operands decoded exactly; f32 accumulate)",
        "data": "synthetic",
        "config": {"workload": "Qwen3-30B-A3B-shaped MoE layer: NVFP4 W4A4 forward + BF16 dgrad + dense W4A4 QKV",
                   "tokens": T, "hidden": H, "experts": E, "topk": k, "intermediate": I,
                   "qkv_n": S.qkv_n, "routing": args.routing, "routed_rows": Rr,
                   "parallelism": "single GPU"},
        "layer_tokens_per_s": round(T / (ms_step * 1e-3), 1),
        "graph": graph,
        "per_op": per_op,
        "roofline": roofline,
        "setup_s": round(setup_s, 1),
    }

    # the other routings of the gate_up workload (uniform k-subsets, Zipf(1.2)):
    # the same step, timed the same way, after the headline's
    by_routing = {args.routing: {"ms_per_step": round(ms_step, 4), "value": round(value, 2),
                                 "gate_up_gemm": per_op["gate_up_gemm"], "down_gemm": per_op["down_gemm"]}}
    for kind in ("softmax", "uniform", "zipf"):
        if kind == args.routing or args.single_routing:
            continue
        set_routing(kind)
        ms_k, om_k = timed_steps(min(args.warmup, 5))
        po = per_op_of(om_k)
        by_routing[kind] = {"ms_per_step": round(ms_k, 4), "value": round(w4(om_k), 2),
                            "gate_up_gemm": po["gate_up_gemm"], "down_gemm": po["down_gemm"]}
    by_routing["how"] = "each routing: warm-up steps, then --steps timed steps with per-op HIP events"
    result["by_routing"] = by_routing
    set_routing(args.routing)
    # the same step with the weighted SwiGLU in the gate_up GEMM's epilogue (FP32)
    # and the light FP32-row quantiser in place of the float64 SwiGLU-quantise pass
    ms_f, om_f = timed_steps(min(args.warmup, 5), ops_fused)
    result["fused_swiglu_step"] = {
        "ms_per_step": round(ms_f, 4), "layer_tokens_per_s": round(T / (ms_f * 1e-3), 1),
        "gate_up_gemm_swiglu_us": round(om_f["gate_up_gemm_swiglu"] * 1e3, 2),
        "quantize_h_us": round(om_f["quantize_h"] * 1e3, 2),
        "plain_gate_up_gemm_plus_swiglu_quantize_us": round((op_ms["gate_up_gemm"] + op_ms["swiglu_quantize"]) * 1e3, 2),
        "how": "warm-up steps, then --steps timed steps, after the headline routing's; same buffers"}
    step()
    torch.cuda.synchronize()

    result["practical_ceiling"] = practical_ceiling(gu_tf, per_op["quantize_permute"]["GBps"],
                                                    op_bytes["quantize_permute"])
    if not args.no_comparisons:
        result["comparisons"] = comparisons(
            dict(x=x, dy=dy, ids=ids, E=E, k=k, I=I, H=H, perm=perm, wgu=wgu, wd=wd, dgu=dgu, dh=dh, ws=ws,
                 q_gu=q_gu, q_d=q_d, tw=tw, gu=gu, a2=a2, hbuf=hbuf, fws=fws, dn=dn, dx_perm=dx_perm),
            gemm_flops)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(x_bits, ids_np, wgu_bits, S, args.cpu_seconds)
    print(json.dumps(result), flush=True)


_FLUSH = None


def time_cold(fn, reps):
    """Average µs of one launch of fn, each launch preceded (outside its events)
    by a 512 MiB device write that evicts the last-level cache."""
    import torch
    global _FLUSH
    if _FLUSH is None:
        _FLUSH = torch.empty(512 * 1024 * 1024 // 4, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for _ in range(2):
        _FLUSH.fill_(1.0)
        fn()
    for st, en in evs:
        _FLUSH.fill_(1.0)
        st.record(stream)
        fn()
        en.record(stream)
    torch.cuda.synchronize()
    return float(np.mean([st.elapsed_time(en) for st, en in evs])) * 1e3


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def graph_steps(step, steps, warmup, T):
    """The same step captured once in a HIP graph and replayed `steps` times
    after `warmup` replays (after the eager timed steps, outside them): the
    whole-step time without the host's launch gaps between the kernels."""
    import torch
    stream = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        step()
    stream.wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for _ in range(warmup):
        g.replay()
    st, en = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    st.record(stream)
    for _ in range(steps):
        g.replay()
    en.record(stream)
    torch.cuda.synchronize()
    ms = st.elapsed_time(en) / steps
    return {"ms_per_step": round(ms, 4), "layer_tokens_per_s": round(T / (ms * 1e-3), 1),
            "how": "one step captured in a HIP graph, replayed; same ops, buffers and stream"}


def _time_op(fn, reps=10):
    """Average µs of one launch of fn: 3 untimed, then reps timed on the launch stream."""
    import torch
    stream = torch.cuda.current_stream()
    for _ in range(3):
        fn()
    st, en = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    st.record(stream)
    for _ in range(reps):
        fn()
    en.record(stream)
    torch.cuda.synchronize()
    return st.elapsed_time(en) * 1e3 / reps


def comparisons(t, gemm_flops):
    """The layer's GEMMs at other precisions and the SwiGLU unfused, timed after the
    timed steps (outside them).  Both sides of every comparison are timed the same
    way (3 untimed + 10 timed back-to-back launches, HIP events on the launch
    stream): back-to-back GEMMs hold the matrix cores busy long enough to lower
    the clock, so these figures run slower than the same kernels inside a step and
    are compared only with each other.
      bf16_forward: the forward's expert GEMMs in BF16 (the precision NVFP4
        replaces) against the step's NVFP4 ones;
      nvfp4_input_gradient: the input gradient's GEMMs in NVFP4 (a lower-precision
        backward: the output gradient quantised and permuted like the forward
        input, the SwiGLU gradient quantised per row, the forward weights
        transposed and quantised along their output dimension once, untimed)
        against the step's BF16 ones;
      fused_swiglu_gate_up: the step's gate_up with the FP32 SwiGLU in its
        epilogue + the FP32-row quantiser, against the plain gate_up GEMM + the
        float64 SwiGLU-quantise pass;
      ep8_shard: one GPU's share of 8-way expert parallelism (16 local experts
        whose rows come from every GPU's tokens, about 2048 each): the step's
        32768 routed rows and the first 16 experts' weights, the 128 experts' row
        counts summed in groups of 8 as the local experts' counts, against the
        step's own expert GEMMs."""
    import torch
    import precision_moe_gemm_amd as pmg
    x, dy, ids, E, k, I, H = t["x"], t["dy"], t["ids"], t["E"], t["k"], t["I"], t["H"]
    perm, off = t["perm"], t["perm"]["expert_offsets"]
    r2t = perm["row_to_tk"]
    a = (perm["codes"], perm["bscales"], perm["rscales"], off)
    a2 = t["a2"]
    R = r2t.numel()
    dev = x.device
    tf = lambda name, us: round(gemm_flops[name] / (us * 1e-6) / 1e12, 1)
    out = {}
    # the step's NVFP4 forward GEMMs, timed as the comparisons are
    us_nv_gu = _time_op(lambda: pmg.nvfp4_grouped_gemm(*a, *t["q_gu"], c=t["gu"]))
    us_nv_dn = _time_op(lambda: pmg.nvfp4_grouped_gemm(a2["codes"], a2["bscales"], a2["rscales"], off, *t["q_d"],
                                                       c=t["dn"]))
    # BF16 forward: gate_up reads the token rows through the routing map, down a BF16 SwiGLU output
    gu_bf = torch.empty(R, 2 * I, dtype=torch.float32, device=dev)
    h16 = t["dgu"][:, :I].contiguous()
    dn_bf = torch.empty(R, H, dtype=torch.float32, device=dev)
    us_gu = _time_op(lambda: pmg.bf16_grouped_gemm_gather(x, r2t, k, off, t["wgu"], pmg.W_NK, c=gu_bf))
    us_dn = _time_op(lambda: pmg.bf16_grouped_gemm(h16, off, t["wd"], pmg.W_NK, c=dn_bf))
    out["bf16_forward"] = {
        "gate_up_gemm": {"us": round(us_gu, 2), "TFLOPs": tf("gate_up_gemm", us_gu)},
        "down_gemm": {"us": round(us_dn, 2), "TFLOPs": tf("down_gemm", us_dn)},
        "nvfp4_gate_up_gemm": {"us": round(us_nv_gu, 2), "TFLOPs": tf("gate_up_gemm", us_nv_gu)},
        "nvfp4_down_gemm": {"us": round(us_nv_dn, 2), "TFLOPs": tf("down_gemm", us_nv_dn)},
        "nvfp4_gemms_speedup": round((us_gu + us_dn) / (us_nv_gu + us_nv_dn), 3)}
    del gu_bf, dn_bf, h16
    # the per-GPU share of 8-way expert parallelism
    counts = (off[1:] - off[:-1]).view(E // 8, 8).sum(dim=1)
    off_s = torch.zeros(E // 8 + 1, dtype=torch.int32, device=dev)
    off_s[1:] = torch.cumsum(counts, 0).to(torch.int32)
    q_gu16 = tuple(v[: E // 8].contiguous() for v in t["q_gu"])
    q_d16 = tuple(v[: E // 8].contiguous() for v in t["q_d"])
    us_s_gu = _time_op(lambda: pmg.nvfp4_grouped_gemm(*a[:3], off_s, *q_gu16, c=t["gu"]))
    us_s_dn = _time_op(lambda: pmg.nvfp4_grouped_gemm(a2["codes"], a2["bscales"], a2["rscales"], off_s, *q_d16,
                                                      c=t["dn"]))
    cnt_h = counts.cpu().numpy()
    out["ep8_shard"] = {
        "gate_up_gemm": {"us": round(us_s_gu, 2), "TFLOPs": tf("gate_up_gemm", us_s_gu)},
        "down_gemm": {"us": round(us_s_dn, 2), "TFLOPs": tf("down_gemm", us_s_dn)},
        "layer_gate_up_gemm_us": round(us_nv_gu, 2), "layer_down_gemm_us": round(us_nv_dn, 2),
        "local_experts": E // 8, "rows_per_local_expert": [int(cnt_h.min()), int(cnt_h.max())]}
    del q_gu16, q_d16
    # NVFP4 input gradient against the step's BF16 dgrad GEMMs
    us_bf_dd = _time_op(lambda: pmg.bf16_grouped_gemm_gather(dy, r2t, k, off, t["wd"], pmg.W_KN, c=t["dh"]))
    us_bf_dg = _time_op(lambda: pmg.bf16_grouped_gemm(t["dgu"], off, t["wgu"], pmg.W_KN, c=t["dx_perm"]))

    def transposed_nvfp4(w):     # [E, out, in] -> quantised [E, in, out] along out, K-tiled
        wt = pmg.bf16_transpose(w)
        c_, b_, s_ = pmg.nvfp4_quantize_rows_tiled(wt.view(-1, wt.shape[2]), wt.shape[1])
        return c_, b_, s_.view(-1, wt.shape[1])
    q_dt, q_gut = transposed_nvfp4(t["wd"]), transposed_nvfp4(t["wgu"])
    torch.cuda.synchronize()
    pdy = {"codes": torch.empty(R, H // 2, dtype=torch.uint8, device=dev),
           "bscales": torch.empty(R, H // 16, dtype=torch.uint8, device=dev),
           "rscales": torch.empty(R, dtype=torch.float32, device=dev),
           "expert_offsets": torch.empty(E + 1, dtype=torch.int32, device=dev),
           "row_to_tk": torch.empty(R, dtype=torch.int32, device=dev),
           "tk_to_row": torch.empty(R, dtype=torch.int32, device=dev)}
    g = (torch.empty(R, I, dtype=torch.uint8, device=dev), torch.empty(R, I // 8, dtype=torch.uint8, device=dev),
         torch.empty(R, dtype=torch.float32, device=dev))
    dh = torch.empty(R, I, dtype=torch.float32, device=dev)
    dxp = torch.empty(R, H, dtype=torch.float32, device=dev)
    us_qp = _time_op(lambda: pmg.nvfp4_quantize_permute(dy, ids, E, workspace=t["ws"], out=pdy))
    us_dd = _time_op(lambda: pmg.nvfp4_grouped_gemm(pdy["codes"], pdy["bscales"], pdy["rscales"],
                                                    pdy["expert_offsets"], *q_dt, c=dh))
    us_q = _time_op(lambda: pmg.nvfp4_quantize_rows(t["dgu"], *g))
    us_dg = _time_op(lambda: pmg.nvfp4_grouped_gemm(*g, pdy["expert_offsets"], *q_gut, c=dxp))
    bf = us_bf_dd + us_bf_dg
    total = us_qp + us_dd + us_q + us_dg
    out["nvfp4_input_gradient"] = {
        "grad_quantize_permute": {"us": round(us_qp, 2)},
        "dgrad_down_gemm": {"us": round(us_dd, 2), "TFLOPs": tf("dgrad_down_gemm", us_dd)},
        "swiglu_grad_quantize": {"us": round(us_q, 2)},
        "dgrad_gate_up_gemm": {"us": round(us_dg, 2), "TFLOPs": tf("dgrad_gate_up_gemm", us_dg)},
        "total_us": round(total, 2), "bf16_dgrad_gemms_us": round(bf, 2),
        "speedup_vs_bf16": round(bf / total, 3)}
    del pdy, g, dh, dxp, q_dt, q_gut
    # fused SwiGLU: without the gate/up output (forward only) and with it (kept for the backward)
    fused = lambda gu_out: pmg.nvfp4_grouped_gemm_swiglu(*a, *t["q_gu"], topk_w=t["tw"], row_to_tk=r2t,
                                                         h=t["hbuf"], gu=gu_out, workspace=t["fws"])
    us_f = _time_op(lambda: fused(None))
    us_fg = _time_op(lambda: fused(t["gu"]))
    us_qh = _time_op(lambda: pmg.nvfp4_quantize_rows_f32(t["hbuf"], off, a2["codes"], a2["bscales"], a2["rscales"]))
    us_sq = _time_op(lambda: pmg.swiglu_quantize(t["gu"], off, t["tw"], r2t, out=a2))
    sep = us_nv_gu + us_sq
    out["fused_swiglu_gate_up"] = {
        "gemm_swiglu_us": round(us_f, 2), "gemm_swiglu_with_gu_us": round(us_fg, 2),
        "quantize_h_us": round(us_qh, 2), "plain_gate_up_gemm_us": round(us_nv_gu, 2),
        "swiglu_quantize_f64_us": round(us_sq, 2),
        "speedup_forward_only": round(sep / (us_f + us_qh), 3),
        "speedup_with_gu": round(sep / (us_fg + us_qh), 3)}
    out["nvfp4_weight_gradient"] = weight_gradients(t)
    out["how"] = ("after the timed steps: 3 untimed + 10 timed back-to-back launches per op, HIP events on "
                  "the launch stream, both sides of each comparison alike; same routing, shapes and buffers")
    return out


def weight_gradients(t):
    """The expert weight gradients dW_d[e] = dY_e^T h_e and dW_gu[e] = dGU_e^T x_e in
    NVFP4, quantised along tokens (each operand's per-expert slab, one FP32 scale per
    (expert, channel), E4M3 per 16 tokens; one K-grouped GEMM launch over all
    experts), against BF16 torch.bmm (hipBLASLt) on the same products with every
    expert's tokens zero-padded to the largest expert's count (padding done
    before timing)."""
    import torch
    import precision_moe_gemm_amd as pmg
    x, dy, E, k, I, H = t["x"], t["dy"], t["E"], t["k"], t["I"], t["H"]
    perm = t["perm"]
    off, r2t = perm["expert_offsets"], perm["row_to_tk"]
    R = r2t.numel()
    kofs = pmg.token_blocks(off)
    Kp = pmg.token_capacity(R, E)
    off_h = off.cpu().numpy()
    r2t_l = r2t.long()
    n_max = int(np.diff(off_h).max())
    flops = 2.0 * R * H * I
    res = {}

    def padded(rows):           # [R][C] expert-grouped -> [E][n_max][C], zero rows past each expert
        outp = torch.zeros(E, n_max, rows.shape[1], dtype=torch.bfloat16, device=rows.device)
        for e in range(E):
            o0, o1 = int(off_h[e]), int(off_h[e + 1])
            outp[e, : o1 - o0] = rows[o0:o1].to(torch.bfloat16)
        return outp

    for name, g, g_map, xx, x_map, M, N in (
            ("down", dy, True, t["hbuf"], False, H, I),
            ("gate_up", t["dgu"], False, x, True, 2 * I, H)):
        gq = pmg.nvfp4_quantize_tokens(g, off, kofs, Kp, pmg.W_ROWMAJOR, row_to_tk=r2t if g_map else None, k=k)
        xq = pmg.nvfp4_quantize_tokens(xx, off, kofs, Kp, pmg.W_KTILED, row_to_tk=r2t if x_map else None, k=k)
        dw = torch.empty(E, M, N, dtype=torch.float32, device=x.device)
        dw16 = torch.empty(E, M, N, dtype=torch.bfloat16, device=x.device)
        us_g = _time_op(lambda: pmg.nvfp4_quantize_tokens(g, off, kofs, Kp, pmg.W_ROWMAJOR,
                                                          row_to_tk=r2t if g_map else None, k=k,
                                                          out=dict(zip(("codes", "bscales", "rscales"), gq))))
        us_x = _time_op(lambda: pmg.nvfp4_quantize_tokens(xx, off, kofs, Kp, pmg.W_KTILED,
                                                          row_to_tk=r2t if x_map else None, k=k,
                                                          out=dict(zip(("codes", "bscales", "rscales"), xq))))
        us_mm = _time_op(lambda: pmg.nvfp4_grouped_gemm_wgrad(gq, xq, kofs, c=dw))
        us_mm16 = _time_op(lambda: pmg.nvfp4_grouped_gemm_wgrad(gq, xq, kofs, c=dw16))
        del dw, dw16, gq, xq
        g_rows = g[r2t_l // k] if g_map else g
        x_rows = xx[r2t_l // k] if x_map else xx
        gp = padded(g_rows).transpose(1, 2).contiguous()          # [E][M][n_max]
        xp = padded(x_rows)                                        # [E][n_max][N]
        del g_rows, x_rows
        dwb = torch.empty(E, M, N, dtype=torch.bfloat16, device=x.device)
        us_bf = _time_op(lambda: torch.bmm(gp, xp, out=dwb))
        del gp, xp, dwb
        total = us_g + us_x + us_mm16
        res[name] = {"quantize_grad_us": round(us_g, 2), "quantize_input_us": round(us_x, 2),
                     "gemm_f32_out_us": round(us_mm, 2), "gemm_bf16_out_us": round(us_mm16, 2),
                     "gemm_bf16_out_TFLOPs": round(flops / (us_mm16 * 1e-6) / 1e12, 1),
                     "total_bf16_out_us": round(total, 2), "bf16_bmm_padded_us": round(us_bf, 2),
                     "speedup_vs_bf16": round(us_bf / total, 3)}
    res["padded_tokens_per_expert"] = n_max
    return res


def practical_ceiling(gate_up_tflops, qp_gbps, qp_bytes):
    """Rates the device sustains, measured after the timed steps (outside them):
    FP16 MFMA issue with no memory traffic (the library's MFMA-only kernel), a
    512 MiB device-to-device copy, and a copy that moves the quantize-permute's
    algorithmic bytes (half read, half written) timed like it (cold, HIP events
    around one launch); the headline kernels as fractions of these."""
    import torch
    import precision_moe_gemm_amd as pmg
    st, en = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    iters = 20000
    sink, flops = pmg.mfma_ceiling(iters)
    for _ in range(3):
        pmg.mfma_ceiling(iters, sink)
    st.record()
    for _ in range(5):
        pmg.mfma_ceiling(iters, sink)
    en.record()
    torch.cuda.synchronize()
    mfma_tf = 5 * flops / (st.elapsed_time(en) * 1e-3) / 1e12
    n = 512 * 1024 * 1024 // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    st.record()
    for _ in range(10):
        b.copy_(a)
    en.record()
    torch.cuda.synchronize()
    copy_gbs = 10 * 2 * n * 4 / (st.elapsed_time(en) * 1e-3) / 1e9
    del a, b
    m = int(qp_bytes) // 8                  # floats copied: 4 m bytes read + 4 m written
    a2 = torch.ones(m, dtype=torch.float32, device="cuda")
    b2 = torch.empty_like(a2)
    small_us = time_cold(lambda: b2.copy_(a2), 20)
    small_gbs = 8 * m / (small_us * 1e-6) / 1e9
    return {"mfma_f16_tflops": round(mfma_tf, 1), "copy_gbps": round(copy_gbs, 1),
            "gate_up_frac_of_mfma": round(gate_up_tflops / mfma_tf, 4),
            "quantize_permute_frac_of_copy": round(qp_gbps / copy_gbs, 4),
            "copy_of_quantize_permute_bytes": {"bytes": 8 * m, "us": round(small_us, 2),
                                               "GBps": round(small_gbs, 1),
                                               "frac_hbm_peak": round(small_gbs / 8000.0, 4)},
            "quantize_permute_frac_of_same_bytes_copy": round(qp_gbps / small_gbs, 4),
            "how": "MFMA: 256 workgroups x 8 wavefronts of back-to-back 32x32x16 f16 MFMAs on registers; "
                   "copy: 512 MiB device-to-device, read + write bytes; copy of the quantize-permute's "
                   "bytes: one device-to-device copy launch after a 512 MiB cache-evicting write"}


def cpu_baseline(x_bits, ids, wgu_bits, S, budget_s):
    """The oracle (as it is) on a bounded sample of the same workload, on the host cores.

    Sample: the oracle's quantize-permute of all 4096 tokens, then its gate_up
    grouped GEMM (exact dequantisation, FP64 BLAS on all cores) for the routed
    rows of experts 0, 1, ... until the time budget is used.  The oracle's
    weight quantisation is preparation and is not timed (as on the GPU).
    """
    from oracle import gemm as og, layer as ol, quantize as oq
    threads = len(os.sched_getaffinity(0))
    t = time.time()
    (off, r2t, t2r), a = ol.quantize_permute_ref(x_bits, ids, S.E)
    qp_s = time.time() - t
    Rr = int(off[-1])
    qp_bytes = S.T * S.H * 2 + S.T * S.k * 4 + Rr * (S.H // 2 + S.H // 16 + 4 + 8)
    flops, g_s, e = 0.0, 0.0, 0
    while e < S.E and g_s < budget_s:
        w = oq.quantize_rows_bf16(wgu_bits[e])
        rows = np.arange(off[e], off[e + 1])
        t = time.time()
        if rows.size:
            og.grouped_gemm_ref(a[0][rows], a[1][rows], a[2][rows], np.array([0, rows.size]),
                                *(v[None] for v in w))
            flops += 2.0 * rows.size * S.H * 2 * S.I
        g_s += time.time() - t
        e += 1
    return {"value": round(flops / g_s / 1e12, 6), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"oracle gate_up grouped GEMM over the routed rows of experts 0..{e - 1} "
                      f"({int(off[e] - off[0])} of {Rr} rows); oracle quantize-permute of all {S.T} tokens",
            "quantize_permute_GBps": round(qp_bytes / qp_s / 1e9, 4),
            "cpu": cpu_model(), "seconds": round(g_s + qp_s, 2)}


if __name__ == "__main__":
    main()
