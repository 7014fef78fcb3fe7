#!/usr/bin/env python3
"""Benchmark of the routed 2-bit MoE FFN layer on one MI355X.

A step is one pass of the whole layer (route -> permute -> routed experts +
shared expert -> combine) over one batch of synthetic input.  The default
workload is decode at batch 1: hidden 4096, 256 routed experts, top-8,
intermediate 2048, one bf16 shared expert (intermediate 2048), bf16
activations, 1000 seeded tokens, one token per step.  Each token runs on one of
several device copies of the layer (cycled), so consecutive tokens cannot
reuse each other's weights from the 256 MB last-level cache; a real model's
consecutive tokens through one layer are separated by all its other layers.

Prints ONE JSON line (rank 0).  Timed region: exactly --steps steps,
captured once in a HIP graph and replayed, bracketed by device
synchronizations; inputs and weights are resident in HBM before it starts.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2500.0
METRIC = "routed-MoE layer tokens/sec at decode B=1 and prefill; % of HBM/MFMA peak"
PREFILL_SAMPLE = 8        # tokens per prefill workload checked against the oracle in the same run


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=1000)
    p.add_argument("--warmup", type=int, default=50)
    p.add_argument("--layers", type=int, default=6, help="device copies of the layer, cycled per token")
    p.add_argument("--kernel-reps", type=int, default=0, help="launches per kernel timing pass (default: steps)")
    p.add_argument("--cpu-seconds", type=float, default=12.0, help="budget of the oracle CPU baseline")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-prefill", action="store_true", help="skip the prefill measurements")
    p.add_argument("--prefill-reps", type=int, default=5)
    p.add_argument("--no-q4k", action="store_true", help="skip the 4-bit (q4k) routed-expert workloads")
    p.add_argument("--verify-steps", type=int, default=334, help="steps of the 3-token verify micro-batch")
    p.add_argument("--no-sweep", action="store_true", help="skip the 2/4/8-token verify micro-batches")
    p.add_argument("--probe-gemm", action="store_true",
                   help="hardware-counter probe: --kernel-reps eager launches of the prefill gate/up grouped GEMM "
                        "on the first 2048-token chunk of the long prompt")
    p.add_argument("--probe", action="store_true",
                   help="hardware-counter probe: --kernel-reps eager launches of the decode gate/up kernel over "
                        "cycled layer copies, then one 1 GiB device-to-device copy (the reference for scaling "
                        "the traffic counters); prints one JSON line")
    return p.parse_args()


# HBM traffic of one decode gate/up launch, from rocprofv3 FETCH_SIZE and
# WRITE_SIZE counters on that kernel, each scaled by the same counter's reading
# for a 1 GiB device-to-device copy in the same process.  Valid only for the
# kernel source it was measured on (sha256 of csrc/ffn_gemv.hip).
GATEUP_TRAFFIC = {"src_sha256": "f4b1dcfa1d47c2bf0de63f1e510da51312e672d2f2f28d0a4d97301a8a870775", "bytes": 68494893}


def gemv_source_sha():
    import hashlib
    with open(os.path.join(ROOT, "bit_quantized_moe_permute_amd", "csrc", "ffn_gemv.hip"), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def probe(args):
    """Eager launches only, for counter collection (no timing)."""
    import torch

    import synth
    from bit_quantized_moe_permute_amd import moe_expert_gate_up, moe_route
    from bit_quantized_moe_permute_amd.layer import DeviceLayer, LayerBuffers

    dev = torch.device("cuda:0")
    sp = synth.SPECS["decode"]
    H, E, k = sp.hidden, sp.n_experts, sp.top_k
    L = synth.make_layer(sp)
    layers = [DeviceLayer.from_synth(L, device=dev)]
    for _ in range(args.layers - 1):
        layers.append(layers[0].clone())
    x_np = synth.activations("decode", synth.TOKENS["decode"], H, True)
    x = torch.from_numpy(x_np.view(np.int16)).view(torch.bfloat16).to(dev)
    reps = args.kernel_reps or 50
    b = LayerBuffers.allocate(layers[0], 1)
    for i in range(reps):
        Li = layers[i % args.layers]
        xi = x[i: i + 1]
        moe_route(xi, Li.w_router, E, k, b.topk_idx, b.topk_w, b.offsets, b.perm, b.active, b.ws_route)
        moe_expert_gate_up(Li.desc, xi, b.topk_idx, b.offsets, b.perm, b.active, b.ws_ffn)
    src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    src.fill_(1)
    dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"probe": "decode gate/up", "launches": reps, "copy_bytes": 1 << 30,
                      "gemv_src_sha256": gemv_source_sha()}), flush=True)


def probe_gemm(args):
    """Eager launches of the prefill gate/up grouped GEMM (first 2048-token chunk of the long prompt, one layer
    copy), for counter collection (no timing)."""
    import torch

    import synth
    from bit_quantized_moe_permute_amd import moe_expert_gate_up, moe_route
    from bit_quantized_moe_permute_amd.layer import DeviceLayer, LayerBuffers

    L = synth.make_layer(synth.SPECS["decode"])
    DL = DeviceLayer.from_synth(L)
    T = 2048
    x = torch.from_numpy(synth.activations("long", T, L.spec.hidden, True).view(np.int16)).view(torch.bfloat16).cuda()
    b = LayerBuffers.allocate(DL, T)
    moe_route(x, DL.w_router, DL.E, DL.k, b.topk_idx, b.topk_w, b.offsets, b.perm, b.active, b.ws_route)
    reps = args.kernel_reps or 10
    for _ in range(reps):
        moe_expert_gate_up(DL.desc, x, b.topk_idx, b.offsets, b.perm, b.active, b.ws_ffn)
    torch.cuda.synchronize()
    print(json.dumps({"probe": "prefill gate/up grouped GEMM", "tokens": T, "launches": reps}), flush=True)


def graph_steps(step, K, W):
    """Warm up W steps eagerly, capture K steps in one HIP graph, check one
    replay against an eager recomputation of the last step, then time one
    replay.  Returns (wall seconds, event milliseconds)."""
    import torch
    for i in range(W):
        step(i)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        with torch.cuda.graph(g, stream=cap):
            for i in range(K):
                y_last = step(i)
    torch.cuda.synchronize()
    g.replay()                                   # one untimed replay
    torch.cuda.synchronize()
    y_graph = y_last.clone()
    step(K - 1)                                  # eager recomputation of the last step
    torch.cuda.synchronize()
    if not torch.equal(y_graph, y_last):
        raise RuntimeError("graph replay and eager run disagree")
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_start = time.perf_counter()
    ev0.record()
    g.replay()
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    gpu_ms = ev0.elapsed_time(ev1)
    del g
    torch.cuda.synchronize()
    return wall, gpu_ms


def decode_bytes(H, I, E, k, Is):
    """Algorithmic bytes per decode token, per launch family (selected experts only)."""
    iq2x = I * H // 256 * 66
    q2k = H * I // 256 * 84
    gate_up = k * 2 * iq2x + 2 * Is * H * 2 + H * 2 + (k * I * 2 + Is * 4)          # weights, x, h out
    down = k * q2k + H * Is * 2 + (k * I * 2 + Is * 4) + (k * H * 4 + H * 4)         # weights, h in, outputs
    route = E * H * 2 + H * 2
    combine = k * H * 4 + H * 4 + H * 4 + k * 4
    return dict(gate_up=gate_up, down=down, route=route, combine=combine,
                total=gate_up + down + route + combine)


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU; the layer is a single-GPU hot path "
                                   "(multi-GPU expert parallelism is described, not built)", "n_gpus": args.gpus}))
        sys.exit(2)

    if args.probe:
        probe(args)
        return
    if args.probe_gemm:
        probe_gemm(args)
        return

    import torch

    import synth
    from bit_quantized_moe_permute_amd import moe_expert_gate_up, moe_route
    from bit_quantized_moe_permute_amd.layer import DeviceLayer, LayerBuffers, forward

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    sp = synth.SPECS["decode"]
    H, I, E, k, Is = sp.hidden, sp.inter, sp.n_experts, sp.top_k, sp.shared_inter
    K, W = args.steps, args.warmup
    n_tok = synth.TOKENS["decode"]

    log("generating the decode layer (seeded random blocks)")
    t0 = time.time()
    L = synth.make_layer(sp)
    x_np = synth.activations("decode", n_tok, H, True)
    layers = [DeviceLayer.from_synth(L, device=dev)]
    for _ in range(args.layers - 1):
        layers.append(layers[0].clone())
    x = torch.from_numpy(x_np.view(np.int16)).view(torch.bfloat16).to(dev)
    torch.cuda.synchronize()
    log(f"layer ready in {time.time() - t0:.1f}s ({args.layers} device copies)")

    bufs = [LayerBuffers.allocate(layers[0], 1) for _ in range(2)]

    def step(i):
        b = bufs[i % 2]
        forward(layers[i % args.layers], x[i % n_tok: i % n_tok + 1], b)
        return b.y

    log(f"decode: warmup {W} steps, {K} steps captured in a HIP graph")
    wall, gpu_ms = graph_steps(step, K, W)
    ms_per_step = wall * 1e3 / K
    value = K / wall
    log(f"{K} steps: wall {wall * 1e3:.2f} ms, events {gpu_ms:.2f} ms -> {value:.0f} tokens/s")

    # the same decode steps on one layer copy (consecutive tokens may find experts in the 256 MB last-level cache)
    def step1(i):
        b = bufs[i % 2]
        forward(layers[0], x[i % n_tok: i % n_tok + 1], b)
        return b.y

    nwall, _ = graph_steps(step1, K, W)
    no_cycling = {"tokens_per_s": round(K / nwall, 1), "ms_per_step": round(nwall * 1e3 / K, 5), "layer_copies": 1}
    log(f"decode on one layer copy (no cycling): {K / nwall:.0f} tokens/s")

    # speculative-verify micro-batch: 3 independent tokens per step
    vx_np = synth.activations("verify", 3 * args.verify_steps, H, True)
    vx = torch.from_numpy(vx_np.view(np.int16)).view(torch.bfloat16).to(dev)
    vbufs = [LayerBuffers.allocate(layers[0], 3) for _ in range(2)]

    def vstep(i):
        b = vbufs[i % 2]
        forward(layers[i % args.layers], vx[3 * i: 3 * i + 3], b)
        return b.y

    vK = args.verify_steps
    vwall, _ = graph_steps(vstep, vK, min(W, vK))
    verify = {"tokens_per_step": 3, "steps": vK, "tokens_per_s": round(3 * vK / vwall, 1),
              "us_per_step": round(vwall * 1e6 / vK, 2)}
    log(f"verify: {vK} steps of 3 tokens -> {3 * vK / vwall:.0f} tokens/s, {vwall * 1e6 / vK:.1f} us/step")

    # verifier micro-batches of M = 1 + drafts tokens (independent seeded tokens, same layer copies)
    sweep = {}
    for M in (() if args.no_sweep else (2, 4, 8)):
        mx = torch.from_numpy(synth.activations("verify", M * vK, H, True, seed=12 + M).view(np.int16)) \
            .view(torch.bfloat16).to(dev)
        mbufs = [LayerBuffers.allocate(layers[0], M) for _ in range(2)]

        def mstep(i, M=M, mx=mx, mbufs=mbufs):
            b = mbufs[i % 2]
            forward(layers[i % args.layers], mx[M * i: M * i + M], b)
            return b.y

        mwall, _ = graph_steps(mstep, vK, min(W, vK))
        sweep[f"M{M}"] = {"tokens_per_s": round(M * vK / mwall, 1), "us_per_step": round(mwall * 1e6 / vK, 2)}
        log(f"verify M={M}: {M * vK / mwall:.0f} tokens/s, {mwall * 1e6 / vK:.1f} us/step")
    verify["sweep"] = sweep

    # directional steering of the FFN output (y -= F v (v . y)), fused into the combine
    steer_v = synth.steer_direction(H)
    for Lc in layers:
        Lc.set_steering(steer_v, 1.0)
    swall, _ = graph_steps(step, K, W)
    for Lc in layers:
        Lc.set_steering(None)
    steer = {"tokens_per_s": round(K / swall, 1), "ms_per_step": round(swall * 1e3 / K, 5),
             "combine": combine_bench(k, H, (1, 3, 2048), args.kernel_reps or 200)}
    log(f"decode with steering: {K / swall:.0f} tokens/s; combine kernels {steer['combine']}")

    # dominant kernel: gate/up (+SwiGLU) GEMV, routed and shared rows in one launch
    reps = args.kernel_reps or K
    log(f"timing the gate/up kernel over {reps} launches")
    rb = [LayerBuffers.allocate(layers[0], 1) for _ in range(2)]
    # per-token routing results, computed once (untimed)
    ridx = torch.empty(reps, k, dtype=torch.int32, device=dev)
    roff = torch.empty(reps, E + 1, dtype=torch.int32, device=dev)
    rperm = torch.empty(reps, k, dtype=torch.int32, device=dev)
    ract = torch.empty(reps, E + 1, dtype=torch.int32, device=dev)
    rw = torch.empty(reps, k, dtype=torch.float32, device=dev)
    b0 = rb[0]
    for i in range(reps):
        Li = layers[i % args.layers]
        moe_route(x[i % n_tok: i % n_tok + 1], Li.w_router, E, k, ridx[i], rw[i], roff[i], rperm[i], ract[i],
                  b0.ws_route, bias=Li.bias)
    torch.cuda.synchronize()
    g2 = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        with torch.cuda.graph(g2, stream=cap):
            for i in range(reps):
                Li = layers[i % args.layers]
                moe_expert_gate_up(Li.desc, x[i % n_tok: i % n_tok + 1], ridx[i], roff[i], rperm[i], ract[i],
                                   rb[i % 2].ws_ffn)
    torch.cuda.synchronize()
    g2.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    g2.replay()
    e1.record()
    torch.cuda.synchronize()
    gu_us = e0.elapsed_time(e1) * 1e3 / reps
    nbytes = decode_bytes(H, I, E, k, Is)
    achieved = nbytes["gate_up"] / (gu_us * 1e-6) / 1e9
    log(f"gate/up kernel: {gu_us:.2f} us/launch, {achieved:.0f} GB/s algorithmic")

    traffic = GATEUP_TRAFFIC["bytes"] if GATEUP_TRAFFIC["src_sha256"] == gemv_source_sha() else None
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                "kernel": "k_gemv_gateup_mfma (routed iq2x gate/up on fp8 x fp4 MFMA + bf16 shared gate/up, fused SwiGLU)",
                "bytes_per_launch": nbytes["gate_up"], "avg_launch_us": round(gu_us, 3)}
    step_bw = nbytes["total"] / (ms_per_step * 1e-3) / 1e9

    del g2
    torch.cuda.synchronize()
    prefill = None
    samples = None if args.no_cpu_baseline else []      # prefill outputs for the oracle check
    if not args.no_prefill:
        prefill = prefill_bench(L, layers[0], args.prefill_reps, ("prefill", "long"), samples)

    decode_q4k = None
    if not args.no_q4k:
        # 4-bit routed experts: decode B=1 over cycled copies, and the long prompt
        del layers[1:]
        torch.cuda.synchronize()
        log("generating the q4k layer (seeded random blocks)")
        L4 = synth.make_layer(synth.SPECS["long_q4k"])
        n4 = max(2, args.layers // 2)
        layers4 = [DeviceLayer.from_synth(L4, device=dev)]
        for _ in range(n4 - 1):
            layers4.append(layers4[0].clone())
        torch.cuda.synchronize()

        def qstep(i):
            b = bufs[i % 2]
            forward(layers4[i % n4], x[i % n_tok: i % n_tok + 1], b)
            return b.y

        qwall, _ = graph_steps(qstep, K, W)
        decode_q4k = {"tokens_per_s": round(K / qwall, 1), "ms_per_step": round(qwall * 1e3 / K, 5),
                      "layer_copies": n4}
        log(f"decode q4k: {K / qwall:.0f} tokens/s")
        if not args.no_prefill:
            prefill.update(prefill_bench(L4, layers4[0], args.prefill_reps, ("long_q4k",), samples))
        del layers4
        torch.cuda.synchronize()

    cpu = None
    if not args.no_cpu_baseline:
        # the GPU layer's outputs for the oracle's sample (one call per token), checked in the same run
        pb = LayerBuffers.allocate(layers[0], 1)
        gy, gi = [], []
        for i in range(200):
            forward(layers[0], x[i: i + 1], pb)
            gy.append(pb.y.cpu().numpy()[0].astype(np.float64))
            gi.append(pb.topk_idx.cpu().numpy()[0].copy())
        cpu = cpu_baseline(L, x_np, args.cpu_seconds, np.array(gy), np.array(gi), samples or ())

    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": K, "warmup": W,
        "ms_per_step": round(ms_per_step, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "decode B=1: hidden 4096, 256 routed experts top-8, intermediate 2048 "
                               "(gate/up iq2x 2.06 bpw, down q2k 2.63 bpw), bf16 shared expert 2048, bf16 router; "
                               f"1000 seeded tokens one per step over {args.layers} cycled layer copies",
                   "global_batch": 1, "seq_len": 1, "parallelism": "single GPU"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "step": {"bytes_per_token": nbytes["total"], "effective_GBps": round(step_bw, 1),
                 "hbm_frac": round(step_bw / HBM_PEAK_GBS, 4), "graph_gpu_ms": round(gpu_ms, 3)},
        "verify": verify,
        "decode_steer": steer,
        "decode_no_cycling": no_cycling,
        "decode_q4k": decode_q4k,
        "prefill": prefill,
    }
    print(json.dumps(out), flush=True)


def combine_bench(k, H, Ts, reps):
    """Average launch time of the combine with and without steering, per token count T (graph of `reps`
    launches, HIP events), and the algorithmic bytes each moves: k + 1 input rows, one output row and k weights
    per token, plus the direction once for the steered form."""
    import torch
    from bit_quantized_moe_permute_amd import moe_combine, moe_combine_steer
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev).manual_seed(5)
    v = torch.randn(H, device=dev, generator=g)
    out = {}
    for T in Ts:
        o = torch.randn(T * k, H, device=dev, generator=g)
        w = torch.rand(T, k, device=dev, generator=g)
        sh = torch.randn(T, H, device=dev, generator=g)
        y = torch.empty(T, H, device=dev)
        nbytes = T * ((k + 2) * H * 4 + k * 4)
        res = {}
        for name, fn in (("plain", lambda: moe_combine(o, w, sh, T, k, H, y)),
                         ("steer", lambda: moe_combine_steer(o, w, sh, T, k, H, v, 1.0, y))):
            fn()
            torch.cuda.synchronize()
            gr = torch.cuda.CUDAGraph()
            cap = torch.cuda.Stream()
            cap.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(cap):
                with torch.cuda.graph(gr, stream=cap):
                    for _ in range(reps):
                        fn()
            torch.cuda.synchronize()
            gr.replay()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            gr.replay()
            e1.record()
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / reps
            b = nbytes + (H * 4 if name == "steer" else 0)
            res[name] = {"us": round(us, 3), "GBps": round(b / (us * 1e-6) / 1e9, 1)}
            del gr
        out[f"T{T}"] = res
    return out


def prefill_bench(L, DL, reps, names, samples=None):
    """Prefill workloads on layer DL: a 512-token chunk with a seeded per-expert
    router bias (skewed expert load, "prefill"), and the 11,709-token long
    prompt in 2048-token chunks (5 x 2048 + 1469; "long" with 2-bit experts,
    "long_q4k" with q4k experts).  Reported per workload:
    tokens/s over the whole prompt, and the gate/up grouped-GEMM stage (fp16
    copy of x + k_gemm_gateup) timed alone with HIP events against the bf16/fp16
    MFMA peak, counting only the useful FLOPs (selected experts, real tokens).
    With a list in samples, the GPU outputs of PREFILL_SAMPLE tokens spread over
    the first chunk are appended to it for the oracle check of the same run."""
    import torch

    import synth
    from bit_quantized_moe_permute_amd import moe_expert_gate_up
    from bit_quantized_moe_permute_amd.layer import LayerBuffers, forward

    sp = L.spec
    H, I, k, Is = sp.hidden, sp.inter, sp.top_k, sp.shared_inter
    out = {}
    shapes = {"prefill": (512, 512), "long": (11709, 2048), "long_q4k": (11709, 2048)}
    for name in names:
        T_total, chunk = shapes[name]
        wspec = synth.SPECS[name]
        _, bias = synth.make_router(wspec)
        DL.bias = None if bias is None else torch.from_numpy(bias).cuda()
        x = synth.activations(name, T_total, H, True)
        xd = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
        chunks = [(c, min(chunk, T_total - c)) for c in range(0, T_total, chunk)]
        bufs = {n: LayerBuffers.allocate(DL, n) for n in sorted({n for _, n in chunks})}

        def prompt():
            for c0, n in chunks:
                forward(DL, xd[c0:c0 + n], bufs[n])

        prompt()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record()
        for _ in range(reps):
            prompt()
        e1.record()
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t0) / reps
        # gate/up stage alone, on the first (largest) chunk
        c0, n = chunks[0]
        b = bufs[n]
        forward(DL, xd[c0:c0 + n], b)
        torch.cuda.synchronize()
        f0, f1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        f0.record()
        for _ in range(reps):
            moe_expert_gate_up(DL.desc, xd[c0:c0 + n], b.topk_idx, b.offsets, b.perm, b.active, b.ws_ffn)
        f1.record()
        torch.cuda.synchronize()
        gu_us = f0.elapsed_time(f1) * 1e3 / reps
        if samples is not None:
            # b.y and b.topk_idx still hold the first chunk's layer outputs (the stage loop rewrites only h)
            rows = np.unique(np.linspace(0, n - 1, PREFILL_SAMPLE).astype(np.int64))
            samples.append({"workload": name, "layer": L, "bias": bias, "rows": (c0 + rows).tolist(),
                            "x": x[c0 + rows], "y": b.y.cpu().numpy()[rows].astype(np.float64),
                            "idx": b.topk_idx.cpu().numpy()[rows]})
        flops = 4.0 * n * k * H * I + 4.0 * n * H * Is
        tflops = flops / (gu_us * 1e-6) / 1e12
        step_flops = 6.0 * T_total * k * H * I + 6.0 * T_total * H * Is
        counts = np.diff(b.offsets.cpu().numpy())
        out[name] = {
            "tokens": T_total, "chunk": chunk, "tokens_per_s": round(T_total / wall, 1),
            "ms_per_prompt": round(wall * 1e3, 4),
            "layer_tflops": round(step_flops / wall / 1e12, 2),
            "gate_up_stage": {"us": round(gu_us, 2), "tokens": n, "flops": flops, "tflops": round(tflops, 2),
                              "peak_tflops": BF16_MFMA_PEAK_TFLOPS,
                              "mfma_frac": round(tflops / BF16_MFMA_PEAK_TFLOPS, 4)},
            "tokens_per_expert": {"min": int(counts.min()), "max": int(counts.max()),
                                  "active": int((counts > 0).sum())},
        }
        log(f"prefill {name}: {T_total / wall:.0f} tokens/s, gate/up stage {gu_us:.1f} us "
            f"({tflops:.0f} TFLOP/s)")
        del bufs
        torch.cuda.synchronize()
    DL.bias = None
    return out


def cpu_baseline(L, x_np, budget_s, gpu_y, gpu_idx, prefill_samples=()):
    """The oracle (binary64, plain C with OpenMP over rows) on a bounded sample of
    decode tokens, one call per token, until the time budget is spent.  The GPU
    layer's outputs for the same tokens (gpu_y, gpu_idx) are checked against the
    oracle's after the timed loop: routing bit-exact, per-token relative L2.
    The prefill samples (sampled tokens of each prefill workload's first chunk,
    with that workload's layer and router bias) are checked the same way,
    outside the timed loop."""
    import oracle
    threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or len(os.sched_getaffinity(0))
    sp = L.spec
    done, outs, t0 = 0, [], time.perf_counter()
    while True:
        xt = x_np[done: done + 1]
        outs.append(oracle.layer(xt, L.w_router, sp.top_k, sp.n_experts, sp.inter, sp.gate_up_fmt, L.gate, L.up,
                                 sp.down_fmt, L.down, L.codebook, bias=L.bias, shared=L.shared))
        done += 1
        el = time.perf_counter() - t0
        if el >= budget_s or done >= min(200, len(gpu_y)):
            break
    log(f"oracle: {done} tokens in {el:.1f}s")
    want = np.concatenate([o["y"] for o in outs])
    err = np.linalg.norm(gpu_y[:done] - want, axis=1) / np.linalg.norm(want, axis=1)
    idx_ok = bool(np.array_equal(gpu_idx[:done], np.concatenate([o["topk_idx"] for o in outs])))
    log(f"parity on the sample: routing exact {idx_ok}, max per-token rel L2 {err.max():.3e}")
    prefill_parity = {}
    for smp in prefill_samples:
        Ls, sps = smp["layer"], smp["layer"].spec
        ys, ids = [], []
        for r in range(len(smp["rows"])):
            o = oracle.layer(smp["x"][r: r + 1], Ls.w_router, sps.top_k, sps.n_experts, sps.inter, sps.gate_up_fmt,
                             Ls.gate, Ls.up, sps.down_fmt, Ls.down, Ls.codebook, bias=smp["bias"], shared=Ls.shared)
            ys.append(o["y"][0])
            ids.append(o["topk_idx"][0])
        ys, ids = np.array(ys), np.array(ids)
        e = np.linalg.norm(smp["y"] - ys, axis=1) / np.linalg.norm(ys, axis=1)
        ok = bool(np.array_equal(smp["idx"], ids))
        prefill_parity[smp["workload"]] = {"tokens": len(smp["rows"]), "rows": smp["rows"], "routing_exact": ok,
                                           "max_rel_l2": float(f"{e.max():.3e}"), "tolerance": 1e-3}
        log(f"parity on {smp['workload']} (tokens {smp['rows']} of its first chunk): routing exact {ok}, "
            f"max per-token rel L2 {e.max():.3e}")
    return {"value": round(done / el, 3), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"first {done} of the 1000 decode tokens, whole layer (route, permute, 8 routed experts, "
                      f"shared expert, combine) in binary64, {el:.1f} s",
            "parity": {"tokens": done, "routing_exact": idx_ok, "max_rel_l2": float(f"{err.max():.3e}"),
                       "tolerance": 1e-3},
            "parity_prefill": prefill_parity}


if __name__ == "__main__":
    main()
