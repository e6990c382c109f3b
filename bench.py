"""Benchmark of the ConvRot W4A8 codebook linear layer on one MI355X.

Main line (the step): one W4A8 layer at M=2048, N=K=4096 -- rotate_quant_act on
bf16 activations [2048, 4096] (N(0,1) with 1% of the columns x20) followed by
w4a8_gemm (decode in LDS, int8 MFMA, fused epilogue, bf16 out).  value = layer
TOPS = 2*M*N*K / wall time per step.  The same run also measures the decode
GEMV sweep (M = 1, 2, 4, 8 on one N=K=4096 layer; each launch reads one of 64
distinct weight copies, 605 MB > the 256 MB Infinity Cache, so weights come from
HBM) and reports weight GB/s against the 8 TB/s HBM peak.

The GEMM's duration comes from HIP events recorded on the launch stream inside the
timed region, on sampled steps: the mean interval of whole steps minus that of
rotate_quant_act alone, both starting from an event before rotate_quant_act (an
event delays the next launch by a few microseconds; the difference cancels it).
Weights are seeded N(0, 0.02^2) fp32 draws, rotated and quantised on the GPU by
quantize_w4 (timed over five calls and reported on its own: it is an offline step,
not part of the layer); activations are seeded synthetic draws.

    python bench.py [--gpus 1] [--steps 400] [--warmup 10] [--no-cpu-baseline]
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, GB/s
INT8_PEAK_TOPS = 5000.0         # MI355X dense int8 MFMA, TOPS
BF16_PEAK_TFLOPS = 2500.0       # MI355X dense bf16 MFMA, TFLOP/s
METRIC = "W4A8 linear TOPS (M=2048) and GEMV weight GB/s (M=1..8), % of roofline"


def weight_bytes(n, k):
    """Algorithmic bytes of one layer's storage: 4-bit codes, one fp8 scale per 16
    weights, fp32 channel scales, the 64-byte codebook."""
    return n * k // 2 + n * k // 16 + 4 * n + 64


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=400)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--gemv-launches", type=int, default=640)
    p.add_argument("--sleep-cycles", type=float, default=4e7,
                   help="GPU spin before a launch batch, so the host can queue the whole batch")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-gemv", action="store_true")
    p.add_argument("--no-training", action="store_true", help="skip the training-path and variant kernels")
    p.add_argument("--no-prefill-shapes", action="store_true", help="skip the M=4096 MLP pair and the M=8192 set")
    p.add_argument("--copy-calibration", action="store_true",
                   help="only run a plain 256 MiB device-to-device copy 5 times (counter calibration)")
    args = p.parse_args()
    if args.steps < 4:
        p.error("--steps must be at least 4 (the GEMM's events sample steps 1 and 3 of every 4)")
    return args


def make_layer(B, w):
    """Quantise an fp32 device weight on the GPU; returns the layer."""
    return B.quantize_w4(w)


def host_copy(layer):
    return (layer.qpacked.cpu().numpy(), layer.srel.cpu().numpy(), layer.s_channel.cpu().numpy(),
            layer.codebook.cpu().numpy())


def event_pairs(torch, n):
    return [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]


def mean_ms(pairs):
    return float(np.mean([a.elapsed_time(b) for a, b in pairs]))


def bench_prefill(args, torch, B, device):
    from bit_codebook_quantized_amd import synth
    M, N, K = 2048, 4096, 4096
    w = torch.from_numpy(synth.gaussian_weight(N, K, seed=synth.seed_for(2, 0, synth.ROLE_WEIGHT))).to(device)
    cb = torch.tensor(B.FIXED_CODEBOOK, dtype=torch.float32, device=device)
    B.quantize_w4(w, cb)                               # warm-up of the quantiser
    pairs = event_pairs(torch, 5)
    torch.cuda.synchronize()
    for a, b in pairs:
        a.record()
        layer = B.quantize_w4(w, cb)
        b.record()
    torch.cuda.synchronize()
    quant_ms = mean_ms(pairs)
    host = host_copy(layer)
    del w
    x_np = synth.activations(M, K, seed=synth.seed_for(2, 0, synth.ROLE_ACT), kind="outliers",
                             outlier_seed=synth.seed_for(2, 0, synth.ROLE_OUTLIER))
    x = torch.from_numpy(x_np).to(torch.bfloat16).to(device)
    xq = torch.empty(M, K, dtype=torch.int8, device=device)
    xs = torch.empty(M, dtype=torch.float32, device=device)
    out = torch.empty(M, N, dtype=torch.bfloat16, device=device)
    rq_call = B.prepared_rotate_quant(x, xq, xs)
    gemm_call = B.prepared_linear("w4a8_gemm", xq, xs, layer, out)

    def step(ev=None, whole=True):
        # ev: an event pair from before rotate_quant_act to after the GEMM (whole) or to
        # after rotate_quant_act (not whole), on the launch stream
        if ev is not None:
            ev[0].record()
        rq_call()
        if ev is not None and not whole:
            ev[1].record()
        gemm_call()
        if ev is not None and whole:
            ev[1].record()

    for _ in range(args.warmup):
        step()
    # The GEMM's duration from events in the timed region: steps 1, 1 + P, 1 + 2P, ...
    # bracket the whole step and steps 1 + P/2, 1 + 3P/2, ... only rotate_quant_act, both
    # from an event before it, so the difference of the two means is the GEMM's time on the
    # stream.  Each event costs the GPU a few microseconds (a marker the next launch waits
    # behind): the difference cancels it, and sampling one step in P/2 keeps it out of the
    # rest (P = 16, or 4 for short runs).  Step 0 is skipped: its events include the host's
    # first launch latency.
    period = 16 if args.steps >= 32 else 4
    whole = {i: event_pairs(torch, 1)[0] for i in range(1, args.steps, period)}
    part = {i: event_pairs(torch, 1)[0] for i in range(1 + period // 2, args.steps, period)}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        if i in whole:
            step(whole[i], True)
        elif i in part:
            step(part[i], False)
        else:
            step()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / args.steps
    gemm_ms = mean_ms(list(whole.values())) - mean_ms(list(part.values()))
    # The same step launched from a HIP graph, after the timed region: 32 steps captured
    # once (kernel nodes only, no memory-set node) and replayed.  A graph of a single step
    # measured slower than direct launches (its replay has a fixed cost per launch), so the
    # graph holds 32.
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(32):
            step()
    graph.replay()
    torch.cuda.synchronize()
    reps = max(1, args.steps // 32)
    t0 = time.perf_counter()
    for _ in range(reps):
        graph.replay()
    torch.cuda.synchronize()
    graph_wall = (time.perf_counter() - t0) / (32 * reps)
    del graph
    # rotate_quant_act alone, after the timed region (an event before it in every step would
    # add a gap to the step)
    rq_ms, _ = timed_launches(torch, [rq_call], 20, int(args.sleep_cycles))
    # the GEMM alone: median of 5 trials of 100 back-to-back launches (one event pair each)
    gemm_med_ms = median_trials(torch, [gemm_call], 100, 5, int(args.sleep_cycles))
    # The same launches on operands that toggle fewer bits: a copy of the layer whose scale
    # bytes are 0 (every decoded weight 0) and all-zero activations.  The instruction stream is
    # identical; at full load the chip's clock follows the operands' switching power, so the
    # difference is what the power budget costs this kernel (outputs of these runs are unused).
    zero_layer = B.W4A8Layer(layer.qpacked, torch.zeros_like(layer.srel), layer.codebook, layer.s_channel)
    xq_zero = torch.zeros_like(xq)
    zw_call = B.prepared_linear("w4a8_gemm", xq, xs, zero_layer, out)
    za_call = B.prepared_linear("w4a8_gemm", xq_zero, xs, layer, out)
    operands = {"random_us": round(gemm_med_ms * 1e3, 2),
                "zero_weights_us": round(median_trials(torch, [zw_call], 100, 5, int(args.sleep_cycles)) * 1e3, 2),
                "zero_activations_us": round(median_trials(torch, [za_call], 100, 5, int(args.sleep_cycles)) * 1e3, 2),
                "note": "w4a8_gemm back to back, median of 5 x 100, same launches on all-zero operands"}
    del zw_call, za_call, zero_layer, xq_zero
    ops = 2.0 * M * N * K
    return dict(M=M, N=N, K=K, wall_s=wall, graph_wall_s=graph_wall, rq_ms=rq_ms, gemm_ms=gemm_ms, gemm_med_ms=gemm_med_ms, ops=ops,
                operands=operands,
                x_np=x_np, host=host, quant_ms=quant_ms,
                rq_bytes=3 * M * K + 4 * M,
                gemm_bytes=weight_bytes(N, K) + M * K + 4 * M + 2 * M * N)


def timed_launches(torch, calls, n, sleep_cycles):
    """Launch calls[i % len(calls)] n times back to back, queued behind a GPU sleep long
    enough for the host to enqueue everything, with one event pair around the whole run
    (an event between launches is a marker the next launch waits behind, which would add
    a few us to every launch).  Returns the mean ms per launch, which includes the gaps
    between consecutive kernels, and the host's enqueue time."""
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    torch.cuda._sleep(sleep_cycles)
    e0.record()
    t0 = time.perf_counter()
    for i in range(n):
        calls[i % len(calls)]()
    enqueue_s = time.perf_counter() - t0
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n, enqueue_s


def median_trials(torch, calls, n, trials, sleep_cycles):
    """Median over `trials` of the mean ms per launch of n back-to-back launches."""
    return float(np.median([timed_launches(torch, calls, n, sleep_cycles)[0] for _ in range(trials)]))


def launch_floor(args, torch, B):
    """A kernel that does nothing, launched back to back like the GEMV sweep: the floor
    any kernel of that grid pays for launch and drain (512 blocks of 256 threads is the
    grid of the N = K = 4096 decode GEMV)."""
    res = {}
    for blocks in (512, 1024):
        call = [lambda b=blocks: B.empty_launch(b, 256)]
        ms = median_trials(torch, call, args.gemv_launches, 3, int(args.sleep_cycles))
        res[f"{blocks}x256_us"] = round(ms * 1e3, 3)
    return res


def bench_prefill_shapes(args, torch, B, device, decode_layers=None):
    """The MLP pair at M = 4096 (up 4096 x 12288 x 3072, down 4096 x 3072 x 12288; bf16
    Student-t activations, nu = 4) and the 64-layer set at M = 8192 (the decode set's
    layers; bf16 N(0, 1) activations drawn on the GPU), each GEMM timed as the median of
    5 trials of back-to-back launches, rotate_quant_act separately."""
    from bit_codebook_quantized_amd import synth
    sleep = int(args.sleep_cycles)
    res = {}
    for name, (M, N, K, li) in {"mlp_up": (4096, 12288, 3072, 0), "mlp_down": (4096, 3072, 12288, 1)}.items():
        w = synth.gaussian_weight_device(N, K, seed=synth.seed_for(3, li, synth.ROLE_WEIGHT), device=device)
        layer = B.quantize_w4(w)
        del w
        x = torch.from_numpy(synth.activations(M, K, seed=synth.seed_for(3, li, synth.ROLE_ACT), kind="student_t")).to(
            torch.bfloat16).to(device)
        xq = torch.empty(M, K, dtype=torch.int8, device=device)
        xs = torch.empty(M, dtype=torch.float32, device=device)
        out = torch.empty(M, N, dtype=torch.bfloat16, device=device)
        rq = B.prepared_rotate_quant(x, xq, xs)
        gm = B.prepared_linear("w4a8_gemm", xq, xs, layer, out)
        rq_ms = median_trials(torch, [rq], 50, 5, sleep)
        g_ms = median_trials(torch, [gm], 100, 5, sleep)
        ops = 2.0 * M * N * K
        res[name] = {"M": M, "N": N, "K": K, "gemm_us": round(g_ms * 1e3, 2),
                     "gemm_TOPS": round(ops / (g_ms * 1e-3) / 1e12, 1),
                     "frac_int8_peak": round(ops / (g_ms * 1e-3) / 1e12 / INT8_PEAK_TOPS, 4),
                     "rotate_quant_act_us": round(rq_ms * 1e3, 2),
                     "layer_TOPS": round(ops / ((g_ms + rq_ms) * 1e-3) / 1e12, 1)}
        del layer, x, xq, xs, out, rq, gm
    if decode_layers:
        M = 8192
        xqs = {}
        for k in sorted({l.in_features for l in decode_layers}):
            x = synth.activations_device(M, k, seed=synth.seed_for(4, 100 + k // 3072, synth.ROLE_ACT), device=device)
            xqs[k] = B.rotate_quant_act(x)
            del x
        outs = {n: torch.empty(M, n, dtype=torch.bfloat16, device=device)
                for n in sorted({l.out_features for l in decode_layers})}
        calls = [B.prepared_linear("w4a8_gemm", *xqs[l.in_features], l, outs[l.out_features]) for l in decode_layers]
        ops = sum(2.0 * M * l.out_features * l.in_features for l in decode_layers)
        set_ms = median_trials(torch, calls, len(calls), 5, sleep) * len(calls)
        res["layer_set_M8192"] = {"layers": len(calls), "M": M, "set_us": round(set_ms * 1e3, 1),
                                  "TOPS": round(ops / (set_ms * 1e-3) / 1e12, 1),
                                  "frac_int8_peak": round(ops / (set_ms * 1e-3) / 1e12 / INT8_PEAK_TOPS, 4)}
        del calls, outs, xqs
    return res


def bench_c0(args, torch, B, device):
    """The smallest configuration, M = 16, N = K = 256 (a correctness shape, reported in us
    only): rotate_quant_act and w4a8_gemm (M > 8), each the median of 5 trials of 100
    back-to-back launches, and the two as one step."""
    from bit_codebook_quantized_amd import synth
    M, N, K = 16, 256, 256
    w = synth.gaussian_weight_device(N, K, seed=synth.seed_for(0, 0, synth.ROLE_WEIGHT), device=device)
    layer = make_layer(B, w)
    x = torch.from_numpy(synth.activations(M, K, seed=synth.seed_for(0, 0, synth.ROLE_ACT))).to(
        torch.bfloat16).to(device)
    xq = torch.empty(M, K, dtype=torch.int8, device=device)
    xs = torch.empty(M, dtype=torch.float32, device=device)
    out = torch.empty(M, N, dtype=torch.bfloat16, device=device)
    rq = B.prepared_rotate_quant(x, xq, xs)
    gm = B.prepared_linear("w4a8_gemm", xq, xs, layer, out)
    sleep = int(args.sleep_cycles) // 4
    rq_ms = median_trials(torch, [rq], 100, 5, sleep)
    gm_ms = median_trials(torch, [gm], 100, 5, sleep)
    step_ms = median_trials(torch, [lambda: (rq(), gm())], 100, 5, sleep)
    return {"M": M, "N": N, "K": K, "rotate_quant_act_us": round(rq_ms * 1e3, 3),
            "gemm_us": round(gm_ms * 1e3, 3), "step_us": round(step_ms * 1e3, 3)}


def bench_gemv(args, torch, B, device):
    from bit_codebook_quantized_amd import synth
    N = K = 4096
    copies = 64
    layers = []
    for c in range(copies):
        w = synth.gaussian_weight_device(N, K, seed=synth.seed_for(1, c, synth.ROLE_WEIGHT), device=device)
        layers.append(make_layer(B, w))
        del w
    res = {}
    sleep = int(args.sleep_cycles)
    for m in (1, 2, 4, 8):
        x = torch.from_numpy(synth.activations(m, K, seed=synth.seed_for(1, m, synth.ROLE_ACT))).to(
            torch.bfloat16).to(device)
        xq = torch.empty(m, K, dtype=torch.int8, device=device)
        xs = torch.empty(m, dtype=torch.float32, device=device)
        out = torch.empty(m, N, dtype=torch.bfloat16, device=device)
        rq = [B.prepared_rotate_quant(x, xq, xs)]
        cold = [B.prepared_linear("w4a8_gemv", xq, xs, layers[c], out) for c in range(copies)]
        # median of 5 trials of back-to-back launches (at least 100 each) over the 64 copies
        per_trial = max(100, args.gemv_launches // 5)
        _, enq = timed_launches(torch, cold, per_trial, sleep)
        cold_ms = median_trials(torch, cold, per_trial, 5, sleep)
        warm_ms, _ = timed_launches(torch, cold[:1], 64, sleep // 4)
        rq_ms, _ = timed_launches(torch, rq, 64, sleep // 4)
        # the whole decode layer: rotate_quant_act + w4a8_gemv, and the one-launch w4a8_gemv_act
        two = [lambda c=c: (rq[0](), cold[c]()) for c in range(copies)]
        two_ms, _ = timed_launches(torch, two, args.gemv_launches, sleep)
        act = [B.prepared_gemv_act(x, layers[c], out) for c in range(copies)]
        act_ms, _ = timed_launches(torch, act, args.gemv_launches, sleep)
        # the 64 copies as independent layers of one w4a8_gemv_grouped launch (605 MB of
        # weights per launch: the kernel's streaming rate at this M without per-launch cost)
        gouts = [torch.empty(m, N, dtype=torch.bfloat16, device=device) for _ in range(copies)]
        grouped = [B.prepared_gemv_grouped([(xq, xs, layers[c], gouts[c]) for c in range(copies)])]
        grp_ms = median_trials(torch, grouped, 10, 5, sleep // 4)
        wb = weight_bytes(N, K)
        res[str(m)] = dict(
            gemv_us=round(cold_ms * 1e3, 3),
            weight_GBps=round(wb / (cold_ms * 1e-3) / 1e9, 1),
            frac=round(wb / (cold_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
            total_GBps=round((wb + m * K + 4 * m + 2 * m * N) / (cold_ms * 1e-3) / 1e9, 1),
            warm_cache_us=round(warm_ms * 1e3, 3),
            warm_cache_weight_GBps=round(wb / (warm_ms * 1e-3) / 1e9, 1),
            rotate_quant_us=round(rq_ms * 1e3, 3),
            layer_two_launches_us=round(two_ms * 1e3, 3),
            layer_gemv_act_us=round(act_ms * 1e3, 3),
            layer_gemv_act_weight_GBps=round(wb / (act_ms * 1e-3) / 1e9, 1),
            host_enqueue_us=round(enq / per_trial * 1e6, 2),
            grouped_64_copies_us=round(grp_ms * 1e3, 1),
            grouped_64_copies_weight_GBps=round(copies * wb / (grp_ms * 1e-3) / 1e9, 1),
            grouped_64_copies_frac=round(copies * wb / (grp_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        )
    return res


def bench_decode_set(args, torch, B, device):
    """The 64-layer decode set at M=1 (16 layers each of 3072x3072, 9216x3072,
    12288x3072, 3072x12288; 1.02 GB of weights, four times the Infinity Cache): one
    w4a8_gemv launch per layer, and one w4a8_gemv_grouped call (one launch for all 64)
    for layers that are independent of each other.  GPU time of the whole set, the median
    of 10 runs."""
    from bit_codebook_quantized_amd import synth
    shapes = [(3072, 3072), (9216, 3072), (12288, 3072), (3072, 12288)]
    items, wbytes = [], 0
    for i in range(64):
        n, k = shapes[i // 16]
        w = synth.gaussian_weight_device(n, k, seed=synth.seed_for(4, i, synth.ROLE_WEIGHT), device=device)
        layer = B.quantize_w4(w)
        del w
        x = torch.from_numpy(synth.activations(1, k, seed=synth.seed_for(4, i, synth.ROLE_ACT))).to(
            torch.bfloat16).to(device)
        xq, xs = B.rotate_quant_act(x)
        out = torch.empty(1, n, dtype=torch.bfloat16, device=device)
        items.append((xq, xs, layer, out))
        wbytes += weight_bytes(n, k)
    single = [B.prepared_linear("w4a8_gemv", xq, xs, layer, out) for xq, xs, layer, out in items]
    grouped = B.prepared_gemv_grouped(items)

    def timed_set(calls, reps):
        pairs = event_pairs(torch, reps)
        torch.cuda.synchronize()
        torch.cuda._sleep(int(args.sleep_cycles))
        for r in range(reps):
            pairs[r][0].record()
            for c in calls:
                c()
            pairs[r][1].record()
        torch.cuda.synchronize()
        return float(np.median([a.elapsed_time(b) for a, b in pairs]))

    timed_set(single, 2)
    timed_set([grouped], 2)
    seq_ms = timed_set(single, 10)
    grp_ms = timed_set([grouped], 10)
    return [it[2] for it in items], {"layers": 64, "M": 1, "weight_bytes": wbytes,
            "per_layer_launches_us": round(seq_ms * 1e3, 1),
            "per_layer_weight_GBps": round(wbytes / (seq_ms * 1e-3) / 1e9, 1),
            "grouped_us": round(grp_ms * 1e3, 1),
            "grouped_weight_GBps": round(wbytes / (grp_ms * 1e-3) / 1e9, 1),
            "grouped_frac": round(wbytes / (grp_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)}


def time_us(torch, call, reps, sleep_cycles):
    """Mean GPU time of one call over `reps` back-to-back launches queued behind a GPU
    sleep (events around the whole run)."""
    call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(sleep_cycles)
    e0.record()
    for _ in range(reps):
        call()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / reps


def bench_training(args, torch, B, device):
    """The training-path and variant kernels on the 4096 x 4096 layer: the
    straight-through backward at M = 2048, code-only requantisation (nearest and
    stochastic), fake quantisation, dequantisation, a rank-64 LoRA merge, and the
    SwiGLU epilogue of the prefill GEMM."""
    from bit_codebook_quantized_amd import synth
    M, N, K = 2048, 4096, 4096
    sleep = int(args.sleep_cycles) // 4
    w = synth.gaussian_weight_device(N, K, seed=synth.seed_for(5, 0, synth.ROLE_WEIGHT), device=device)
    layer = B.quantize_w4(w)
    gen = torch.Generator(device).manual_seed(5)
    w2 = w + torch.randn(N, K, device=device, generator=gen) * 0.004
    u = torch.rand(N, K, device=device, generator=gen)
    grad = torch.randn(M, N, device=device, generator=gen).to(torch.bfloat16)
    gx = torch.empty(M, K, dtype=torch.bfloat16, device=device)
    codes = torch.empty(N, K // 2, dtype=torch.uint8, device=device)
    f32 = torch.empty(N, K, dtype=torch.float32, device=device)
    la = torch.randn(64, K, device=device, generator=gen) * 0.02
    lb = torch.randn(N, 64, device=device, generator=gen) * 0.02
    x = torch.from_numpy(synth.activations(M, K, seed=synth.seed_for(5, 0, synth.ROLE_ACT))).to(
        torch.bfloat16).to(device)
    xq, xs = B.rotate_quant_act(x)
    y_sw = torch.empty(M, N // 2, dtype=torch.bfloat16, device=device)
    y = torch.empty(M, N, dtype=torch.bfloat16, device=device)
    calls = {
        "grad_input": B.prepare("w4a8_grad_input", grad, M, layer.qpacked, layer.srel, layer.codebook,
                                layer.s_channel, N, K, 16, gx),
        "requantize_nearest": lambda: B.requantize_codes(w2, layer, out=codes),
        "requantize_stochastic": lambda: B.requantize_codes(w2, layer, u=u, out=codes),
        "fake_quant": lambda: B.fake_quant(w2, layer, out=f32),
        "dequantize": lambda: B.dequantize(layer, out=f32),
        "lora_merge_r64": lambda: B.lora_merged_weight(layer, la, lb, 0.5, out=f32),
        "gemm_swiglu": B.prepared_linear("w4a8_gemm", xq, xs, layer, y_sw, B.SWIGLU),
        "gemm_plain": B.prepared_linear("w4a8_gemm", xq, xs, layer, y),
    }
    us = {k: time_us(torch, c, 10, sleep) for k, c in calls.items()}
    wb = weight_bytes(N, K)
    fp = N * K * 4
    res = {
        "layer": "4096 x 4096",
        "grad_input": {"M": M, "us": round(us["grad_input"], 1),
                       "TFLOPs": round(2 * M * N * K / us["grad_input"] / 1e6, 1),
                       "frac_bf16_peak": round(2 * M * N * K / us["grad_input"] / 1e6 / BF16_PEAK_TFLOPS, 4)},
    }
    for name, nbytes in [("requantize_nearest", fp + N * K // 2 + N * K // 16),
                         ("requantize_stochastic", 2 * fp + N * K // 2 + N * K // 16),
                         ("fake_quant", 2 * fp + N * K // 16),
                         ("dequantize", wb + fp),
                         ("lora_merge_r64", wb + fp + 2 * 64 * N * 4)]:
        res[name] = {"us": round(us[name], 1), "GBps": round(nbytes / (us[name] * 1e-6) / 1e9, 1),
                     "frac_hbm": round(nbytes / (us[name] * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4)}
    res["gemm_swiglu_epilogue"] = {"M": M, "us": round(us["gemm_swiglu"], 2),
                                   "plain_gemm_us": round(us["gemm_plain"], 2)}
    return res


def cpu_baseline(pre, min_seconds=10.0):
    """The oracle, untuned, on the host cores: the M=2048 layer step split into its four
    steps (rotate + quantise, int8-grid decode, exact fp64-BLAS contraction, epilogue),
    each repeated until it has run for a share of ``min_seconds``; whole-step TOPS from
    the sum of the four per-call times."""
    import oracle as O
    x = pre["x_np"]
    packed, srel, sch, cb = pre["host"]
    M, N, K = pre["M"], pre["N"], pre["K"]
    xq, xs = O.rotate_quant_act(x)
    w8 = O.decode_w4(packed, srel, cb)
    acc = O.gemm_exact(xq, w8)
    steps = {"rotate_quant_act": lambda: O.rotate_quant_act(x),
             "decode_w4": lambda: O.decode_w4(packed, srel, cb),
             "gemm_exact_fp64_blas": lambda: O.gemm_exact(xq, w8),
             "epilogue_bf16": lambda: O.epilogue(acc, xs, sch, out="bf16")}
    share = {"rotate_quant_act": 0.2, "decode_w4": 0.15, "gemm_exact_fp64_blas": 0.5, "epilogue_bf16": 0.15}
    per_call, detail = {}, {}
    for name, fn in steps.items():
        reps, t0 = 0, time.perf_counter()
        while True:
            fn()
            reps += 1
            dt = time.perf_counter() - t0
            if dt >= min_seconds * share[name] or reps >= 200:
                break
        per_call[name] = dt / reps
        detail[name] = {"s_per_call": round(dt / reps, 4), "reps": reps}
    detail["rotate_quant_act"]["GBps"] = round((3 * M * K + 4 * M) / per_call["rotate_quant_act"] / 1e9, 2)
    detail["decode_w4"]["GBps"] = round((N * K // 2 + N * K // 16 + N * K) / per_call["decode_w4"] / 1e9, 2)
    detail["gemm_exact_fp64_blas"]["TOPS"] = round(2.0 * M * N * K / per_call["gemm_exact_fp64_blas"] / 1e12, 4)
    detail["epilogue_bf16"]["GBps"] = round((8 * M * N + 4 * M + 4 * N + 2 * M * N) / per_call["epilogue_bf16"] / 1e9, 2)
    total = sum(per_call.values())
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count()
    blas, threads = "unknown", None
    try:
        from threadpoolctl import threadpool_info
        infos = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if infos:
            blas = f"{infos[0].get('internal_api')} {infos[0].get('version')}"
            threads = infos[0].get("num_threads")
    except Exception:
        pass
    return {"value": round(2.0 * M * N * K / total / 1e12, 5), "unit": "TOPS",
            "cores": threads if threads else cores, "kind": "oracle",
            "sample": f"the M=2048 N=K=4096 step, its four steps timed separately ({total:.2f} s per step)",
            "host_cores": cores, "blas": blas, "blas_threads": threads, "steps": detail}


GEMM_SRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "bit_codebook_quantized_amd", "csrc",
                        "gemm.hip")
TRAFFIC_FILE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles", "traffic_w4a8_gemm.json")


def measured_traffic():
    """HBM bytes per GEMM launch from the committed counter summary, if it was taken on
    the kernel source as it is now (else None)."""
    import hashlib
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
        with open(GEMM_SRC, "rb") as f:
            src_hash = hashlib.sha256(f.read()).hexdigest()
    except (OSError, ValueError):
        return None
    if rec.get("gemm_source_sha256") != src_hash:
        return None
    return rec.get("hbm_bytes_per_launch")


def copy_calibration():
    import torch
    n = 256 << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": 5}))


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration()
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: --gpus {args.gpus} is not supported (the path shards along N; "
              "this benchmark measures one GPU)", file=sys.stderr)
        sys.exit(2)
    import torch
    from bit_codebook_quantized_amd import w4a8 as B
    B.load()
    device = "cuda:0"
    torch.cuda.set_device(0)

    t_start = time.perf_counter()

    def done(part):   # a progress line on stderr as each part ends (the JSON line stays alone on stdout)
        print(f"bench: {part} done at {time.perf_counter() - t_start:.1f} s", file=sys.stderr, flush=True)

    pre = bench_prefill(args, torch, B, device)
    done("prefill step")
    c0 = bench_c0(args, torch, B, device)
    gemv = None if args.no_gemv else bench_gemv(args, torch, B, device)
    floor = None if args.no_gemv else launch_floor(args, torch, B)
    decode_layers, decode_set = (None, None) if args.no_gemv else bench_decode_set(args, torch, B, device)
    done("decode GEMVs")
    prefill_shapes = None if args.no_prefill_shapes else bench_prefill_shapes(args, torch, B, device, decode_layers)
    del decode_layers
    done("prefill shapes")
    training = None if args.no_training else bench_training(args, torch, B, device)
    done("training-path kernels")
    cpu = None if args.no_cpu_baseline else cpu_baseline(pre)
    done("cpu baseline")

    tops = pre["ops"] / pre["wall_s"] / 1e12
    gemm_tops = pre["ops"] / (pre["gemm_ms"] * 1e-3) / 1e12
    line = {
        "metric": METRIC,
        "value": round(tops, 2),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(pre["wall_s"] * 1e3, 4),
        "graph32_ms_per_step": round(pre["graph_wall_s"] * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": "W4A8 layer prefill M=2048 N=4096 K=4096: rotate_quant_act + w4a8_gemm, "
                               "bf16 activations N(0,1) with 41 outlier columns x20, bf16 output, weight "
                               "N(0,0.02^2) quantised by quantize_w4",
                   "M": pre["M"], "N": pre["N"], "K": pre["K"], "rot_block": 256, "group": 16},
        "roofline": {"bound": "mfma", "achieved": round(gemm_tops, 2), "peak": INT8_PEAK_TOPS,
                     "unit": "TOPS", "frac": round(gemm_tops / INT8_PEAK_TOPS, 4), "traffic": measured_traffic(),
                     "kernel": "w4a8_gemm", "kernel_us": round(pre["gemm_ms"] * 1e3, 3),
                     "kernel_us_median_5x100": round(pre["gemm_med_ms"] * 1e3, 3)},
        "gemm_operand_dependence": pre["operands"],
        "quantize_w4": {"us": round(pre["quant_ms"] * 1e3, 1), "layer": "4096 x 4096 fp32, rotated on the fly",
                        "Mweights_per_s": round(pre["N"] * pre["K"] / (pre["quant_ms"] * 1e-3) / 1e6, 1),
                        "note": "offline weight quantisation, not part of the step"},
        "rotate_quant_act": {"us": round(pre["rq_ms"] * 1e3, 3),
                             "GBps": round(pre["rq_bytes"] / (pre["rq_ms"] * 1e-3) / 1e9, 1),
                             "frac_hbm": round(pre["rq_bytes"] / (pre["rq_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)},
        "c0_step": c0,
        "gemv": gemv,
        "launch_floor": floor,
        "gemv_decode_set": decode_set,
        "prefill_shapes": prefill_shapes,
        "training_and_variants": training,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
