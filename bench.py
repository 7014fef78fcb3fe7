#!/usr/bin/env python3
"""Benchmark of the routed 2-bit MoE FFN layer on one MI355X.

A step is one pass of the whole layer (route -> permute -> routed experts +
shared expert -> combine) over one batch of synthetic input.  The default
workload is decode at batch 1: hidden 4096, 256 routed experts, top-8,
intermediate 2048, one bf16 shared expert (intermediate 2048), bf16
activations, one token per step drawn from a seeded set of 1000.  Each token
runs on one of several device copies of the layer (cycled), so consecutive
tokens cannot reuse each other's weights from the 256 MB last-level cache; a
real model's consecutive tokens through one layer are separated by all its
other layers.

Prints ONE JSON line (rank 0).  Timed region: exactly --steps steps,
captured once in a HIP graph and replayed, bracketed by device
synchronizations; inputs and weights are resident in HBM before it starts.

After the GPU measurements the CPU oracle runs on the host, on the same inputs:
timed (the CPU baseline) and as the parity check of the same run, on every
token of the decode, verify and 512-token prefill workloads, every token of
the long prompt's first chunk, and a covering set of tokens (at least one per
32-token tile of every expert's tokens, and per 32-token tile of the shared
expert) in each other chunk of the long prompt, in both expert formats.
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
TILE = 32                 # token fragment of the grouped-GEMM work items (the cover sets' unit)
TOL = 1e-3                # per-token relative L2 of the layer output


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=1000)
    p.add_argument("--warmup", type=int, default=50)
    p.add_argument("--layers", type=int, default=6, help="device copies of the layer, cycled per token")
    p.add_argument("--kernel-reps", type=int, default=0, help="launches per kernel timing pass (default: max(steps, 200))")
    p.add_argument("--cpu-seconds", type=float, default=10.0, help="budget of the per-token oracle timing")
    p.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle (timing and parity)")
    p.add_argument("--no-prefill", action="store_true", help="skip the prefill measurements")
    p.add_argument("--prefill-reps", type=int, default=5)
    p.add_argument("--no-q4k", action="store_true", help="skip the 4-bit (q4k) routed-expert workloads")
    p.add_argument("--verify-steps", type=int, default=334, help="steps of the 3-token verify micro-batch")
    p.add_argument("--no-sweep", action="store_true", help="skip the 2/4/8-token verify micro-batches")
    p.add_argument("--probe-gemm", action="store_true",
                   help="hardware-counter probe: --kernel-reps eager launches of the prefill gate/up and down "
                        "grouped GEMMs on the first 2048-token chunk of the long prompt, then one 1 GiB copy")
    p.add_argument("--probe", action="store_true",
                   help="hardware-counter probe: --kernel-reps eager decode steps (route, gate/up, down) over "
                        "cycled layer copies, then one 1 GiB device-to-device copy (the reference for scaling "
                        "the traffic counters); prints one JSON line")
    return p.parse_args()


# HBM traffic of one decode gate/up launch, from rocprofv3 FETCH_SIZE and
# WRITE_SIZE counters on that kernel, each scaled by the same counter's reading
# for a 1 GiB device-to-device copy in the same process.  Valid only for the
# kernel source it was measured on (sha256 of csrc/ffn_gemv.hip).
GATEUP_TRAFFIC = {"src_sha256": "87d3aae657e9d8c827bd0c80070712ac34f277906d8e010f05ab66038bb8506c", "bytes": 68558261}


def gemv_source_sha():
    import hashlib
    with open(os.path.join(ROOT, "bit_quantized_moe_permute_amd", "csrc", "ffn_gemv.hip"), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def to_dev(x_np):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x_np).view(np.int16)).view(torch.bfloat16).cuda()


def copy_reference():
    """One 1 GiB device-to-device copy: the known-size reference the traffic counters are scaled by."""
    import torch
    src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    dst.copy_(src)
    torch.cuda.synchronize()


def probe(args):
    """Eager decode steps only (route, gate/up, down), for counter collection (no timing)."""
    import torch

    import synth
    from bit_quantized_moe_permute_amd import moe_expert_down, moe_expert_gate_up, moe_route
    from bit_quantized_moe_permute_amd.layer import DeviceLayer, LayerBuffers

    sp = synth.SPECS["decode"]
    H, E, k = sp.hidden, sp.n_experts, sp.top_k
    L = synth.make_layer(sp)
    layers = [DeviceLayer.from_synth(L)]
    for _ in range(args.layers - 1):
        layers.append(layers[0].clone())
    x = to_dev(synth.activations("decode", synth.TOKENS["decode"], H, True))
    reps = args.kernel_reps or 50
    b = LayerBuffers.allocate(layers[0], 1)
    for i in range(reps):
        Li = layers[i % args.layers]
        xi = x[i: i + 1]
        moe_route(xi, Li.w_router, E, k, b.topk_idx, b.topk_w, b.offsets, b.perm, b.active, b.ws_route)
        moe_expert_gate_up(Li.desc, xi, b.topk_idx, b.offsets, b.perm, b.active, b.ws_ffn)
        moe_expert_down(Li.desc, xi, b.topk_idx, b.offsets, b.perm, b.active, b.slot_out, b.shared_out, b.ws_ffn)
    torch.cuda.synchronize()
    copy_reference()
    print(json.dumps({"probe": "decode route, gate/up, down", "launches": reps, "copy_bytes": 1 << 30,
                      "gemv_src_sha256": gemv_source_sha()}), flush=True)


def probe_gemm(args):
    """Eager launches of the prefill grouped GEMMs (gate/up, then down) on the first 2048-token chunk of the long
    prompt, one layer copy, for counter collection (no timing)."""
    import torch

    import synth
    from bit_quantized_moe_permute_amd import moe_expert_down, moe_expert_gate_up, moe_route
    from bit_quantized_moe_permute_amd.layer import DeviceLayer, LayerBuffers

    L = synth.make_layer(synth.SPECS["decode"])
    DL = DeviceLayer.from_synth(L)
    T = 2048
    x = to_dev(synth.activations("long", T, L.spec.hidden, True))
    b = LayerBuffers.allocate(DL, T)
    moe_route(x, DL.w_router, DL.E, DL.k, b.topk_idx, b.topk_w, b.offsets, b.perm, b.active, b.ws_route)
    reps = args.kernel_reps or 10
    for _ in range(reps):
        moe_expert_gate_up(DL.desc, x, b.topk_idx, b.offsets, b.perm, b.active, b.ws_ffn)
        moe_expert_down(DL.desc, x, b.topk_idx, b.offsets, b.perm, b.active, b.slot_out, b.shared_out, b.ws_ffn)
    torch.cuda.synchronize()
    copy_reference()
    print(json.dumps({"probe": "prefill gate/up and down grouped GEMMs", "tokens": T, "launches": reps,
                      "copy_bytes": 1 << 30}), flush=True)


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


def graph_time_us(launch, reps):
    """Average duration in microseconds of launch(i) for i < reps, captured back to back in one HIP graph and
    timed with HIP events on the stream that replays it (after one untimed replay)."""
    import torch
    launch(0)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        with torch.cuda.graph(g, stream=cap):
            for i in range(reps):
                launch(i)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    g.replay()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / reps
    del g
    torch.cuda.synchronize()
    return us


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


def stream_read_peak(nbytes, reps=200):
    """Measured streaming-read rate (GB/s) of the library's plain read kernel at `nbytes` per launch: reps
    launches over distinct, consecutive windows of a 4 GiB buffer (so no launch finds its bytes in the 256 MB
    last-level cache), best of five grid sizes."""
    import torch
    from bit_quantized_moe_permute_amd import moe_probe_stream_read
    span = 4 << 30
    nbytes = (nbytes + 255) // 256 * 256
    buf = torch.empty(span, dtype=torch.uint8, device="cuda")
    buf.fill_(3)
    best = None
    for blocks in (1024, 2048, 4096, 8192, 16384):
        sink = torch.zeros(blocks, dtype=torch.int32, device="cuda")
        n_win = span // nbytes

        def launch(i, blocks=blocks, sink=sink, n_win=n_win):
            off = (i % n_win) * nbytes
            moe_probe_stream_read(buf[off: off + nbytes], nbytes, sink, blocks)

        us = graph_time_us(launch, reps)
        gbs = nbytes / (us * 1e-6) / 1e9
        if best is None or gbs > best["GBps"]:
            best = {"GBps": round(gbs, 1), "us": round(us, 3), "bytes": nbytes, "workgroups": blocks}
    del buf
    torch.cuda.synchronize()
    return best


def cover_tokens(idx, perm, offsets, k):
    """Greedy cover of a chunk's work items by tokens: every TILE-token fragment of every expert's tokens (in
    permutation order, as the grouped GEMM tiles them) and every TILE-token tile of the shared expert holds at
    least one chosen token.  Returns the chosen token indices, ascending."""
    T = idx.shape[0]
    E = offsets.shape[0] - 1
    pos_item = np.empty(T * k, dtype=np.int64)          # permutation position -> routed item
    n_items = 0
    for e in range(E):
        n = int(offsets[e + 1] - offsets[e])
        if n:
            pos_item[offsets[e]: offsets[e + 1]] = n_items + np.arange(n) // TILE
            n_items += (n + TILE - 1) // TILE
    inv = np.empty(T * k, dtype=np.int64)
    inv[perm] = np.arange(T * k)
    tok_items = np.concatenate([pos_item[inv].reshape(T, k), (n_items + np.arange(T) // TILE)[:, None]], axis=1)
    n_items += (T + TILE - 1) // TILE
    covered = np.zeros(n_items, dtype=bool)
    chosen = []
    while not covered.all():
        gain = (~covered[tok_items]).sum(axis=1)
        t = int(np.argmax(gain))
        chosen.append(t)
        covered[tok_items[t]] = True
    return np.array(sorted(chosen), dtype=np.int64)


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
    from bit_quantized_moe_permute_amd import moe_combine, moe_expert_down, moe_expert_gate_up, moe_route
    from bit_quantized_moe_permute_amd.layer import DeviceLayer, LayerBuffers, forward, forward_layer

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
    x = to_dev(x_np)
    torch.cuda.synchronize()
    log(f"layer ready in {time.time() - t0:.1f}s ({args.layers} device copies)")

    bufs = [LayerBuffers.allocate(layers[0], 1) for _ in range(2)]

    def step(i):
        b = bufs[i % 2]
        forward_layer(layers[i % args.layers], x[i % n_tok: i % n_tok + 1], b)
        return b.y

    log(f"decode: warmup {W} steps, {K} steps captured in a HIP graph")
    wall, gpu_ms = graph_steps(step, K, W)
    ms_per_step = wall * 1e3 / K
    value = K / wall
    log(f"{K} steps: wall {wall * 1e3:.2f} ms, events {gpu_ms:.2f} ms -> {value:.0f} tokens/s")

    # the same steps as the three calls moe_route, moe_expert_ffn, moe_combine (routing in two launches)
    def step3(i):
        b = bufs[i % 2]
        forward(layers[i % args.layers], x[i % n_tok: i % n_tok + 1], b)
        return b.y

    twall, _ = graph_steps(step3, K, W)
    three_calls = {"tokens_per_s": round(K / twall, 1), "ms_per_step": round(twall * 1e3 / K, 5)}
    log(f"decode as three calls: {K / twall:.0f} tokens/s")

    # the same decode steps on one layer copy (consecutive tokens may find experts in the 256 MB last-level cache)
    def step1(i):
        b = bufs[i % 2]
        forward_layer(layers[0], x[i % n_tok: i % n_tok + 1], b)
        return b.y

    nwall, _ = graph_steps(step1, K, W)
    no_cycling = {"tokens_per_s": round(K / nwall, 1), "ms_per_step": round(nwall * 1e3 / K, 5), "layer_copies": 1}
    log(f"decode on one layer copy (no cycling): {K / nwall:.0f} tokens/s")

    # per-call latency: eager moe_layer calls enqueued back to back (no host sync in between), a HIP event pair on
    # the launch stream around each; the spread of single-token GPU times, graph launch not involved
    n_lat = min(K, 1000)
    cs = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_lat)]
    for i in range(W):
        step(i)
    torch.cuda.synchronize()
    for i in range(n_lat):
        evs[i][0].record(cs)
        step(i)
        evs[i][1].record(cs)
    torch.cuda.synchronize()
    lat = sorted(a.elapsed_time(b) * 1e3 for a, b in evs)
    latency = {"calls": n_lat, "p50_us": round(lat[n_lat // 2], 2),
               "p99_us": round(lat[min(n_lat - 1, (99 * n_lat) // 100)], 2), "max_us": round(lat[-1], 2),
               "method": "HIP event pair on the launch stream around each eager one-token moe_layer call"}
    log(f"decode per-call latency (eager): p50 {latency['p50_us']} us, p99 {latency['p99_us']} us")

    # speculative-verify micro-batch: 3 independent tokens per step
    vK = args.verify_steps
    vx_np = synth.activations("verify", 3 * vK, H, True)
    vx = to_dev(vx_np)
    vbufs = [LayerBuffers.allocate(layers[0], 3) for _ in range(2)]

    def vstep(i):
        b = vbufs[i % 2]
        forward_layer(layers[i % args.layers], vx[3 * i: 3 * i + 3], b)
        return b.y

    vwall, _ = graph_steps(vstep, vK, min(W, vK))
    verify = {"tokens_per_step": 3, "steps": vK, "tokens_per_s": round(3 * vK / vwall, 1),
              "us_per_step": round(vwall * 1e6 / vK, 2)}
    log(f"verify: {vK} steps of 3 tokens -> {3 * vK / vwall:.0f} tokens/s, {vwall * 1e6 / vK:.1f} us/step")

    # verifier micro-batches of M = 1 + drafts tokens (independent seeded tokens, same layer copies)
    sweep = {}
    for M in (() if args.no_sweep else (2, 4, 8)):
        mx = to_dev(synth.activations("verify", M * vK, H, True, seed=12 + M))
        mbufs = [LayerBuffers.allocate(layers[0], M) for _ in range(2)]

        def mstep(i, M=M, mx=mx, mbufs=mbufs):
            b = mbufs[i % 2]
            forward_layer(layers[i % args.layers], mx[M * i: M * i + M], b)
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
    reps = args.kernel_reps or max(K, 200)
    steer = {"tokens_per_s": round(K / swall, 1), "ms_per_step": round(swall * 1e3 / K, 5),
             "combine": combine_bench(k, H, (1, 3, 2048), reps)}
    log(f"decode with steering: {K / swall:.0f} tokens/s; combine kernels {steer['combine']}")

    # each decode kernel family alone: graphs of `reps` launches over the cycled layer copies
    log(f"timing the decode kernels over {reps} launches each")
    rb = [LayerBuffers.allocate(layers[0], 1) for _ in range(2)]
    ridx = torch.empty(reps, k, dtype=torch.int32, device=dev)
    roff = torch.empty(reps, E + 1, dtype=torch.int32, device=dev)
    rperm = torch.empty(reps, k, dtype=torch.int32, device=dev)
    ract = torch.empty(reps, E + 1, dtype=torch.int32, device=dev)
    rw = torch.empty(reps, k, dtype=torch.float32, device=dev)

    def t_route(i):
        Li = layers[i % args.layers]
        moe_route(x[i % n_tok: i % n_tok + 1], Li.w_router, E, k, ridx[i], rw[i], roff[i], rperm[i], ract[i],
                  rb[i % 2].ws_route, bias=Li.bias)

    def t_gate_up(i):
        Li = layers[i % args.layers]
        moe_expert_gate_up(Li.desc, x[i % n_tok: i % n_tok + 1], ridx[i], roff[i], rperm[i], ract[i],
                           rb[i % 2].ws_ffn)

    def t_down(i):
        Li = layers[i % args.layers]
        b = rb[i % 2]
        moe_expert_down(Li.desc, x[i % n_tok: i % n_tok + 1], ridx[i], roff[i], rperm[i], ract[i], b.slot_out,
                        b.shared_out, b.ws_ffn)

    def t_combine(i):
        b = rb[i % 2]
        moe_combine(b.slot_out, rw[i], b.shared_out, 1, k, H, b.y)

    route_us = graph_time_us(t_route, reps)           # also fills ridx .. ract for the kernels below
    gu_us = graph_time_us(t_gate_up, reps)
    down_us = graph_time_us(t_down, reps)
    comb_us = graph_time_us(t_combine, reps)
    nbytes = decode_bytes(H, I, E, k, Is)
    achieved = nbytes["gate_up"] / (gu_us * 1e-6) / 1e9
    log(f"decode kernels: route {route_us:.2f}, gate/up {gu_us:.2f} ({achieved:.0f} GB/s), down {down_us:.2f}, "
        f"combine {comb_us:.2f} us/launch")
    peak_gu = stream_read_peak(nbytes["gate_up"])
    peak_down = stream_read_peak(nbytes["down"])
    log(f"streaming-read ceiling: {peak_gu['GBps']:.0f} GB/s at {nbytes['gate_up']} B, "
        f"{peak_down['GBps']:.0f} GB/s at {nbytes['down']} B")

    traffic = GATEUP_TRAFFIC["bytes"] if GATEUP_TRAFFIC["src_sha256"] == gemv_source_sha() else None
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                "kernel": "k_gemv_gateup_mfma (routed iq2x gate/up on fp8 x fp4 MFMA + bf16 shared gate/up, fused SwiGLU)",
                "bytes_per_launch": nbytes["gate_up"], "avg_launch_us": round(gu_us, 3),
                "peak_measured": peak_gu["GBps"], "frac_measured": round(achieved / peak_gu["GBps"], 4),
                "peak_measured_by": "plain streaming-read kernel at the same bytes per launch, cycled over 4 GiB"}
    down_gbs = nbytes["down"] / (down_us * 1e-6) / 1e9
    decode_kernels = {
        "route_us": round(route_us, 3), "gate_up_us": round(gu_us, 3), "down_us": round(down_us, 3),
        "combine_us": round(comb_us, 3), "sum_us": round(route_us + gu_us + down_us + comb_us, 3),
        "gate_up_GBps": round(achieved, 1), "down_GBps": round(down_gbs, 1),
        "down_frac": round(down_gbs / HBM_PEAK_GBS, 4), "down_frac_measured": round(down_gbs / peak_down["GBps"], 4),
        "stream_read_gate_up_bytes": peak_gu, "stream_read_down_bytes": peak_down,
        "bytes_per_token": nbytes,
    }
    step_bw = nbytes["total"] / (ms_per_step * 1e-3) / 1e9
    del rb
    torch.cuda.synchronize()

    keep = not args.no_cpu_baseline
    prefill, samples = None, {}
    if not args.no_prefill:
        prefill = prefill_bench(L, layers[0], args.prefill_reps, ("prefill", "long"), samples if keep else None)

    # GPU outputs of every decode token (one call each) and every verify step (three tokens per call) on the
    # first layer copy, for the oracle check of the same run
    dec_gpu = ver_gpu = None
    if keep:
        dec_gpu = collect(layers[0], x, 1)
        ver_gpu = collect(layers[0], vx, 3)

    decode_q4k, L4 = None, None
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
            forward_layer(layers4[i % n4], x[i % n_tok: i % n_tok + 1], b)
            return b.y

        qwall, _ = graph_steps(qstep, K, W)
        decode_q4k = {"tokens_per_s": round(K / qwall, 1), "ms_per_step": round(qwall * 1e3 / K, 5),
                      "layer_copies": n4}
        log(f"decode q4k: {K / qwall:.0f} tokens/s")
        if not args.no_prefill:
            prefill.update(prefill_bench(L4, layers4[0], args.prefill_reps, ("long_q4k",), samples if keep else None))
        del layers4
        torch.cuda.synchronize()

    cpu = None
    if keep:
        cpu = oracle_leg(args, L, L4, x_np, vx_np, dec_gpu, ver_gpu, samples)

    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": K, "warmup": W,
        "ms_per_step": round(ms_per_step, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "decode B=1: hidden 4096, 256 routed experts top-8, intermediate 2048 "
                               "(gate/up iq2x 2.06 bpw, down q2k 2.63 bpw), bf16 shared expert 2048, bf16 router; "
                               f"{K} timed steps of one seeded token each (tokens 0..{min(K, n_tok) - 1} of a "
                               f"1000-token set, cycling past 1000), over {args.layers} cycled layer copies",
                   "global_batch": 1, "seq_len": 1, "parallelism": "single GPU", "timed_tokens": K},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "step": {"bytes_per_token": nbytes["total"], "effective_GBps": round(step_bw, 1),
                 "hbm_frac": round(step_bw / HBM_PEAK_GBS, 4), "graph_gpu_ms": round(gpu_ms, 3)},
        "decode_kernels": decode_kernels,
        "decode_three_calls": three_calls,
        "verify": verify,
        "decode_steer": steer,
        "decode_no_cycling": no_cycling,
        "decode_latency": latency,
        "decode_q4k": decode_q4k,
        "prefill": prefill,
    }
    print(json.dumps(out), flush=True)


def collect(DL, xd, T):
    """Layer outputs of consecutive T-token calls over all rows of xd (device bf16 [N][H]) on layer DL: routing,
    weights, slot, shared and layer outputs as host arrays."""
    import torch
    from bit_quantized_moe_permute_amd.layer import LayerBuffers, forward_layer
    N, H = xd.shape
    steps = N // T
    b = LayerBuffers.allocate(DL, T)
    y = torch.empty(steps * T, H, dtype=torch.float32, device=xd.device)
    slot = torch.empty(steps * T * DL.k, H, dtype=torch.float32, device=xd.device)
    sh = torch.empty(steps * T, H, dtype=torch.float32, device=xd.device)
    idx = torch.empty(steps * T, DL.k, dtype=torch.int32, device=xd.device)
    tw = torch.empty(steps * T, DL.k, dtype=torch.float32, device=xd.device)
    for s in range(steps):
        r = slice(s * T, (s + 1) * T)
        forward_layer(DL, xd[r], b)
        y[r].copy_(b.y)
        slot[s * T * DL.k: (s + 1) * T * DL.k].copy_(b.slot_out)
        sh[r].copy_(b.shared_out)
        idx[r].copy_(b.topk_idx)
        tw[r].copy_(b.topk_w)
    torch.cuda.synchronize()
    return {"y": y.cpu().numpy(), "slot": slot.cpu().numpy(), "shared": sh.cpu().numpy(), "idx": idx.cpu().numpy(),
            "w": tw.cpu().numpy(), "tokens_per_call": T}


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
        for name, fn in (("plain", lambda i: moe_combine(o, w, sh, T, k, H, y)),
                         ("steer", lambda i: moe_combine_steer(o, w, sh, T, k, H, v, 1.0, y))):
            us = graph_time_us(fn, reps)
            b = nbytes + (H * 4 if name == "steer" else 0)
            res[name] = {"us": round(us, 3), "GBps": round(b / (us * 1e-6) / 1e9, 1)}
        out[f"T{T}"] = res
    return out


def prefill_bench(L, DL, reps, names, samples=None):
    """Prefill workloads on layer DL: a 512-token chunk with a seeded per-expert
    router bias (skewed expert load, "prefill"), and the 11,709-token long
    prompt in 2048-token chunks (5 x 2048 + 1469; "long" with 2-bit experts,
    "long_q4k" with q4k experts).  Reported per workload:
    tokens/s over the whole prompt, and the gate/up and down grouped-GEMM
    stages timed alone with HIP events on the first chunk, against the bf16/fp16
    MFMA peak, counting only the useful FLOPs (selected experts, real tokens).
    With a dict in samples, each chunk's GPU outputs for the tokens the oracle
    checks in the same run are stored under samples[name]: every token of the
    512-token chunk and of the long prompt's first 2-bit chunk, a covering set
    of tokens (cover_tokens) of every other chunk."""
    import torch

    import synth
    from bit_quantized_moe_permute_amd import moe_expert_down, moe_expert_gate_up
    from bit_quantized_moe_permute_amd.layer import LayerBuffers, forward_layer

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
        xd = to_dev(x)
        chunks = [(c, min(chunk, T_total - c)) for c in range(0, T_total, chunk)]
        bufs = {n: LayerBuffers.allocate(DL, n) for n in sorted({n for _, n in chunks})}

        def prompt():
            for c0, n in chunks:
                forward_layer(DL, xd[c0:c0 + n], bufs[n])

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
        # gate/up and down stages alone, on the first (largest) chunk
        c0, n = chunks[0]
        b = bufs[n]
        forward_layer(DL, xd[c0:c0 + n], b)
        torch.cuda.synchronize()
        xc = xd[c0:c0 + n]
        gu_us = graph_time_us(lambda i: moe_expert_gate_up(DL.desc, xc, b.topk_idx, b.offsets, b.perm, b.active,
                                                           b.ws_ffn), reps)
        dn_us = graph_time_us(lambda i: moe_expert_down(DL.desc, xc, b.topk_idx, b.offsets, b.perm, b.active,
                                                        b.slot_out, b.shared_out, b.ws_ffn), reps)
        counts = np.diff(b.offsets.cpu().numpy())
        gu_flops = 4.0 * n * k * H * I + 4.0 * n * H * Is
        dn_flops = 2.0 * n * k * H * I + 2.0 * n * H * Is
        step_flops = 6.0 * T_total * k * H * I + 6.0 * T_total * H * Is
        gu_tf = gu_flops / (gu_us * 1e-6) / 1e12
        dn_tf = dn_flops / (dn_us * 1e-6) / 1e12
        out[name] = {
            "tokens": T_total, "chunk": chunk, "tokens_per_s": round(T_total / wall, 1),
            "ms_per_prompt": round(wall * 1e3, 4),
            "layer_tflops": round(step_flops / wall / 1e12, 2),
            "gate_up_stage": {"us": round(gu_us, 2), "tokens": n, "flops": gu_flops, "tflops": round(gu_tf, 2),
                              "peak_tflops": BF16_MFMA_PEAK_TFLOPS,
                              "mfma_frac": round(gu_tf / BF16_MFMA_PEAK_TFLOPS, 4)},
            "down_stage": {"us": round(dn_us, 2), "tokens": n, "flops": dn_flops, "tflops": round(dn_tf, 2),
                           "peak_tflops": BF16_MFMA_PEAK_TFLOPS, "mfma_frac": round(dn_tf / BF16_MFMA_PEAK_TFLOPS, 4)},
            "tokens_per_expert": {"min": int(counts.min()), "max": int(counts.max()),
                                  "active": int((counts > 0).sum())},
        }
        log(f"prefill {name}: {T_total / wall:.0f} tokens/s, gate/up stage {gu_us:.1f} us ({gu_tf:.0f} TFLOP/s), "
            f"down stage {dn_us:.1f} us ({dn_tf:.0f} TFLOP/s)")
        if sp.down_fmt == 2:
            # the approximate fast mode (opt-in): q2k down weights as one fp16 fused multiply-add each, the shared
            # expert's h in one bf16 plane; checked against the oracle at 5e-3 by the test suite
            from bit_quantized_moe_permute_amd import PRECISION_FAST
            fdesc = DL.make_desc(precision=PRECISION_FAST)

            def prompt_fast():
                for c0_, n_ in chunks:
                    forward_layer(DL, xd[c0_:c0_ + n_], bufs[n_], desc=fdesc)

            prompt_fast()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(reps):
                prompt_fast()
            torch.cuda.synchronize()
            fwall = (time.perf_counter() - t0) / reps
            forward_layer(DL, xc, b, desc=fdesc)
            fdn_us = graph_time_us(lambda i: moe_expert_down(fdesc, xc, b.topk_idx, b.offsets, b.perm, b.active,
                                                             b.slot_out, b.shared_out, b.ws_ffn), reps)
            out[name]["fast_mode"] = {"tokens_per_s": round(T_total / fwall, 1), "ms_per_prompt": round(fwall * 1e3, 4),
                                      "speedup": round(wall / fwall, 3), "down_stage_us": round(fdn_us, 2),
                                      "tolerance": 5e-3}
            log(f"prefill {name} fast mode: {T_total / fwall:.0f} tokens/s ({wall / fwall:.2f}x), down stage "
                f"{fdn_us:.1f} us")
            forward_layer(DL, xc, b)
            torch.cuda.synchronize()
        if samples is not None:
            rows_all = []
            for ci, (c0, n) in enumerate(chunks):
                bb = bufs[n]
                forward_layer(DL, xd[c0:c0 + n], bb)
                torch.cuda.synchronize()
                idx = bb.topk_idx.cpu().numpy()
                full = name == "prefill" or (name == "long" and ci == 0)
                rows = np.arange(n) if full else cover_tokens(idx, bb.perm.cpu().numpy(), bb.offsets.cpu().numpy(), k)
                rt = torch.from_numpy(rows).cuda()
                srows = (rt[:, None] * k + torch.arange(k, device="cuda")[None, :]).reshape(-1)
                rows_all.append({"chunk": ci, "c0": c0, "n": n, "full": full, "rows": rows, "x": x[c0 + rows],
                                 "idx": idx[rows], "w": bb.topk_w.cpu().numpy()[rows],
                                 "y": bb.y[rt].cpu().numpy(), "slot": bb.slot_out[srows].cpu().numpy(),
                                 "shared": bb.shared_out[rt].cpu().numpy()})
            samples[name] = {"layer": L, "bias": bias, "chunks": rows_all}
            log(f"prefill {name}: kept {sum(len(c['rows']) for c in rows_all)} tokens' outputs for the oracle check")
        del bufs
        torch.cuda.synchronize()
    DL.bias = None
    return out


# ----------------------------------------------------------------------------
# the oracle on the host: CPU baseline and parity of the same run
# ----------------------------------------------------------------------------
def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def oracle_call(Ls, x_rows, bias):
    import oracle
    sps = Ls.spec
    return oracle.layer(x_rows, Ls.w_router, sps.top_k, sps.n_experts, sps.inter, sps.gate_up_fmt, Ls.gate, Ls.up,
                        sps.down_fmt, Ls.down, Ls.codebook, bias=bias, shared=Ls.shared)


def compare(gpu, ref):
    """GPU rows against oracle rows: routing bit-exact, weights within 1e-6, per-token / per-slot relative L2."""
    def rel(g, w):
        g = g.reshape(w.shape[0], -1).astype(np.float64)
        w = w.reshape(w.shape[0], -1)
        den = np.linalg.norm(w, axis=1)
        return np.linalg.norm(g - w, axis=1) / np.where(den > 0, den, 1.0)
    e_y = rel(gpu["y"], ref["y"])
    e_s = rel(gpu["slot"], ref["slot_out"])
    e_h = rel(gpu["shared"], ref["shared_out"])
    idx_ok = bool(np.array_equal(gpu["idx"], ref["topk_idx"]))
    w_err = float(np.abs(gpu["w"].astype(np.float64) - ref["topk_w"]).max())
    ok = idx_ok and w_err <= 1e-6 and max(e_y.max(), e_s.max(), e_h.max()) <= TOL
    return {"tokens": int(e_y.shape[0]), "routing_exact": idx_ok, "max_abs_weight_err": float(f"{w_err:.3e}"),
            "max_rel_l2": float(f"{e_y.max():.3e}"), "max_rel_l2_slot": float(f"{e_s.max():.3e}"),
            "max_rel_l2_shared": float(f"{e_h.max():.3e}"), "tolerance": TOL, "pass": bool(ok)}


def rows_of(d, rows, k):
    rows = np.asarray(rows)
    srows = (rows[:, None] * k + np.arange(k)[None, :]).reshape(-1)
    return {"y": d["y"][rows], "slot": d["slot"][srows], "shared": d["shared"][rows], "idx": d["idx"][rows],
            "w": d["w"][rows]}


def timed_calls(Ls, x, T, budget_s, limit):
    """Oracle on consecutive T-token calls over x until the time budget is spent (at least one call, at most
    `limit` tokens); returns (outputs per call, tokens done, seconds)."""
    outs, done, t0 = [], 0, time.perf_counter()
    while done + T <= min(limit, x.shape[0]):
        outs.append(oracle_call(Ls, x[done: done + T], Ls.bias))
        done += T
        if time.perf_counter() - t0 >= budget_s:
            break
    return outs, done, time.perf_counter() - t0


def merge(outs):
    return {key: np.concatenate([o[key] for o in outs]) for key in ("y", "slot_out", "shared_out", "topk_idx", "topk_w")}


def oracle_leg(args, L, L4, x_np, vx_np, dec_gpu, ver_gpu, samples):
    """The oracle (binary64, plain C with OpenMP over rows) on the host:
    - timing: decode one token per call and verify three tokens per call on a bounded sample of each (the CPU
      baseline is the decode rate), one thread on two decode tokens, the 512-token prefill chunk in one call, the
      long prompt's first 2048-token chunk in one call (whole prompt extrapolated from it), and the q4k long
      prompt's cover-set tokens in one call (extrapolated from that rate);
    - parity: the same calls' outputs plus one batched call over the rest of each workload, against the GPU
      outputs of the same tokens."""
    import oracle
    threads = oracle.get_threads()
    k = L.spec.top_k
    res = {"cpu_model": cpu_model(), "threads": threads, "configs": {}, "parity": {}}
    # one thread, two decode tokens
    oracle.set_threads(1)
    t0 = time.perf_counter()
    for i in range(2):
        oracle_call(L, x_np[i: i + 1], None)
    t1 = time.perf_counter() - t0
    oracle.set_threads(threads)
    res["one_thread"] = {"tokens_per_s": round(2 / t1, 3), "sample": "decode tokens 0 and 1, one call each"}
    log(f"oracle, one thread: {2 / t1:.2f} tokens/s")

    # decode: one token per call (timed), then the rest of the 1000 tokens batched
    outs, done, dec_s = timed_calls(L, x_np, 1, args.cpu_seconds, len(x_np))
    value = done / dec_s
    log(f"oracle decode: {done} tokens one per call in {dec_s:.1f}s ({value:.2f} tokens/s, {threads} threads)")
    ref = merge(outs)
    if done < len(x_np):
        ref = merge([ref, oracle_call(L, x_np[done:], None)])
    res["parity"]["decode"] = compare(dec_gpu, ref)
    log(f"parity decode (all {len(x_np)} tokens): {res['parity']['decode']}")

    # verify: three tokens per call (timed), then the rest batched
    vouts, vdone, vel = timed_calls(L, vx_np, 3, args.cpu_seconds / 2, len(vx_np))
    res["configs"]["verify"] = {"tokens_per_s": round(vdone / vel, 3), "steps": vdone // 3, "s": round(vel, 2),
                                "sample": f"first {vdone // 3} verify steps, three tokens per call"}
    vref = merge(vouts)
    nv = 3 * (len(vx_np) // 3)
    if vdone < nv:
        vref = merge([vref, oracle_call(L, vx_np[vdone:nv], None)])
    res["parity"]["verify"] = compare(ver_gpu, vref)
    log(f"parity verify (all {nv} tokens, 3 per GPU call): {res['parity']['verify']}")

    for name in ("prefill", "long", "long_q4k"):
        if name not in samples:
            continue
        smp = samples[name]
        Ls, bias = smp["layer"], smp["bias"]
        chunks = smp["chunks"]
        parts = []
        if name in ("prefill", "long"):
            c = chunks[0]                                    # a full chunk in one call: timed
            t0 = time.perf_counter()
            r = oracle_call(Ls, c["x"], bias)
            el = time.perf_counter() - t0
            entry = {"tokens": int(c["n"]), "s": round(el, 2), "tokens_per_s": round(c["n"] / el, 3)}
            if name == "long":
                entry["extrapolated_prompt_s"] = round(el * 11709 / c["n"], 1)
                entry["label"] = "extrapolated: the 11,709-token prompt timed as its first 2048-token chunk x 11709/2048"
            res["configs"][name] = entry
            log(f"oracle {name}: {c['n']} tokens in one call, {el:.1f}s")
            parts.append((c, r))
            rest = chunks[1:]
        else:
            rest = chunks
        if rest:
            xs = np.concatenate([c["x"] for c in rest])
            t0 = time.perf_counter()
            r = oracle_call(Ls, xs, bias)
            el = time.perf_counter() - t0
            if name == "long_q4k":
                res["configs"][name] = {
                    "tokens": int(xs.shape[0]), "s": round(el, 2), "tokens_per_s": round(xs.shape[0] / el, 3),
                    "extrapolated_prompt_s": round(el * 11709 / xs.shape[0], 1),
                    "label": "extrapolated: rate on the cover-set tokens of all six chunks in one call x 11709"}
            o = 0
            for c in rest:
                n = len(c["rows"])
                parts.append((c, {key: r[key][o * (k if key == "slot_out" else 1): (o + n) * (k if key == "slot_out" else 1)]
                                  for key in ("y", "slot_out", "shared_out", "topk_idx", "topk_w")}))
                o += n
        per = []
        for c, r in parts:
            cmp_ = compare(c, r)
            cmp_.update({"chunk": c["chunk"], "chunk_tokens": int(c["n"]), "all_tokens": bool(c["full"])})
            per.append(cmp_)
        res["parity"][name] = {
            "chunks": per, "tokens": int(sum(p["tokens"] for p in per)),
            "routing_exact": all(p["routing_exact"] for p in per),
            "max_rel_l2": max(p["max_rel_l2"] for p in per), "max_rel_l2_slot": max(p["max_rel_l2_slot"] for p in per),
            "pass": all(p["pass"] for p in per), "tolerance": TOL,
            "covers": "every token" if all(p["all_tokens"] for p in per) else
                      "every token of the first chunk, then per chunk a token set covering every 32-token tile of "
                      "every expert's tokens and of the shared expert" if name == "long" else
                      "per chunk a token set covering every 32-token tile of every expert's tokens and of the shared "
                      "expert"}
        log(f"parity {name}: {res['parity'][name]['tokens']} tokens, pass {res['parity'][name]['pass']}, "
            f"max rel L2 {res['parity'][name]['max_rel_l2']:.3e}")

    res.update({"value": round(value, 3), "unit": "tokens/s", "cores": threads, "kind": "oracle",
                "sample": f"decode tokens 0..{done - 1}, one call each, whole layer (route, permute, 8 routed "
                          f"experts, shared expert, combine) in binary64, {dec_s:.1f} s"})
    # the documented keys first
    order = ["value", "unit", "cores", "kind", "sample"]
    return {key: res[key] for key in order} | {key: v for key, v in res.items() if key not in order}


if __name__ == "__main__":
    main()
