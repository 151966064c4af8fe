#!/usr/bin/env python3
"""Throughput of the streaming timestep-forcing denoise step on one MI355X.

Default workload (one "step" = one block through one denoise stage): 40 layers,
each with its own bf16 KV ring (window 4 blocks) and 1560-token sink, each layer
running 3D Rolling RoPE (Q, K, sink K), block attention 40 heads x 128 over
Nq = 4680 query tokens and Nk = 1560 + 4*4680 + 4680 = 24960 keys, and the ring
append/evict; then one flow-matching Euler update (dt = -0.25) of a
16x3x60x104 fp32 latent.  Steady state: blocks >= 5 (ring full).  The
one-time sink replacement happens in warm-up at block 1.

All inputs are synthetic N(0,1) tensors resident in HBM before the timed
region (there are no trained weights).  One JSON line goes to stdout; progress
goes to stderr.

Other workloads (--workload): c2 (one 40x128 layer, attention timed alone),
c3 (the same layer with a window of 8 blocks, Nk 43680), c5 (720p-shaped layer, 44x80 tokens per frame, streamed for 1000 blocks:
sustained blocks/s and cache-update GB/s), chain (a complete 4-step denoise of
each block on one GPU: 4 timestep-forcing stages x 40 layers, la_denoise_chain),
c2fp8 (the e4m3 attention kernel alone at the C2 shape), refresh (the NFE-5
clean-cache baseline: 4 attend-only passes and a refresh pass per block).
"""

from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

METRIC = "block-attn TFLOP/s + denoise-step blocks/s at 1 GPU; % bf16 MFMA / HBM peak"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
FRAMES = 3
DELTA = -1
THETA = 10000.0
NOISE = 0.75
DT = -0.25

# Calibrated HBM traffic per attention launch at the C2/C4 shape (Nq 4680, Nk 24960),
# from rocprofv3 FETCH_SIZE/WRITE_SIZE runs scaled by a copy kernel of known size,
# keyed by the attention kernel version the library reports; any other version
# reports null (the counters were taken on a different kernel).
ATTN_TRAFFIC_BYTES = {"attn-v9": 8.618e8}
# The same for the e4m3 attention kernel at the C2 shape (--workload c2fp8).
FP8_TRAFFIC_BYTES = {"fp8-v6": 5.337e+08}


_T0 = time.perf_counter()


def log(msg):
    print(f"[{time.perf_counter() - _T0:7.1f}s] {msg}", file=sys.stderr, flush=True)


def attn_flops(nq, nk, d, h):
    return 4.0 * nq * nk * d * h


# --------------------------------------------------------------------------- GPU
def gpu_step_bench(args, Hl, Wl, W, H, d, n_layers, with_euler=True):
    import torch
    import streaming_causal_video_amd as L

    L.lib()
    dev = "cuda"
    bt, st = FRAMES * Hl * Wl, Hl * Wl
    nk = st + (W + 1) * bt
    gen = torch.Generator(device=dev)
    gen.manual_seed(1234)

    def randn(shape, dtype=torch.bfloat16):
        return torch.randn(shape, device=dev, dtype=torch.float32, generator=gen).to(dtype)

    log(f"setup: {n_layers} layers, Hl={Hl} Wl={Wl} W={W} H={H} d={d}, Nq={bt} Nk={nk}")
    stack = L.KVRingStack(n_layers, W, bt, st, H, d, torch.bfloat16, NOISE)
    for l in range(n_layers):
        stack.sink_k_raw[l].copy_(randn((st, H, d)))
        stack.sink_v[l].copy_(randn((st, H, d)))
    pool = 2
    ins = [[tuple(randn((bt, H, d)) for _ in range(3)) for _ in range(n_layers)] for _ in range(pool)]
    outs = [torch.empty((bt, H, d), dtype=torch.bfloat16, device=dev) for _ in range(n_layers)]
    qws = torch.empty((bt, H, d), dtype=torch.bfloat16, device=dev)
    kws = torch.empty_like(qws)
    sws = torch.empty((st, H, d), dtype=torch.bfloat16, device=dev)
    table = torch.empty(L.la_rope_table_bytes(Hl, Wl, d) // 4, dtype=torch.float32, device=dev)
    L.la_rope_table_fill(table, Hl, Wl, d, THETA)
    aws = L.AttnWorkspace(bt, H) if args.attn_schedule == "balanced" else None
    lat_shape = (16, 3, 60, 104)
    x = torch.randn(lat_shape, device=dev, generator=gen) if with_euler else None
    vels = [torch.randn(lat_shape, device=dev, generator=gen) for _ in range(pool)] if with_euler else None
    torch.cuda.synchronize()

    def step(b, events=None):
        e = b % pool
        q = [ins[e][l][0] for l in range(n_layers)]
        k = [ins[e][l][1] for l in range(n_layers)]
        v = [ins[e][l][2] for l in range(n_layers)]
        skn = [t[:st] for t in k] if b == 1 else None
        svn = [t[:st] for t in v] if b == 1 else None
        L.la_denoise_step(stack.states, b, q, k, v, outs, qws, kws, sws, table, Hl, Wl, FRAMES,
                          DELTA, THETA, scale=d ** -0.5, sink_k_new=skn, sink_v_new=svn, x=x,
                          vel=vels[e] if with_euler else None, dt=DT, timing_events=events,
                          attn_ws=aws)

    # warm-up: block 1 (sink replacement) .. the ring is full after block W
    block = 0
    for _ in range(W + args.warmup):
        block += 1
        step(block)
    torch.cuda.synchronize()
    log(f"warm-up done ({block} blocks)")

    nev = 6 * n_layers + 2
    ev_objs = []
    ev_arrays = []
    for _ in range(args.steps):
        objs = [torch.cuda.Event(enable_timing=True) for _ in range(nev)]
        for o in objs:
            o.record()  # creates the underlying HIP event
        arr = (ctypes.c_void_p * nev)(*[o.cuda_event for o in objs])
        ev_objs.append(objs)
        ev_arrays.append(arr)
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t0.record()
    for i in range(args.steps):
        block += 1
        step(block, ev_arrays[i])
    t1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = t0.elapsed_time(t1)
    ms_step = total_ms / args.steps

    def avg(off):
        vals = [objs[6 * l + off].elapsed_time(objs[6 * l + off + 1])
                for objs in ev_objs for l in range(n_layers)]
        return float(np.mean(vals)), float(np.std(vals))

    rope_ms, _ = avg(0)
    attn_ms, attn_sd = avg(2)
    app_ms, _ = avg(4)
    eul = [objs[6 * n_layers].elapsed_time(objs[6 * n_layers + 1]) for objs in ev_objs]
    log(f"timed {args.steps} steps: {ms_step:.3f} ms/step (host wall {wall / args.steps * 1e3:.3f} ms/step)")
    fl = attn_flops(bt, nk, d, H)
    rope_bytes = 2 * (2 * bt + st) * H * d * 2
    app_bytes = 2 * 2 * bt * H * d * 2
    res = {
        "ms_per_step": ms_step,
        "blocks_per_s": 1e3 / ms_step,
        "attn_ms": attn_ms, "attn_ms_sd": attn_sd,
        "attn_tflops": fl / (attn_ms * 1e-3) / 1e12,
        "attn_flop_per_launch": fl,
        "rope_us": rope_ms * 1e3, "rope_gbs": rope_bytes / (rope_ms * 1e-3) / 1e9,
        "rope_bytes": rope_bytes,
        "append_us": app_ms * 1e3, "append_gbs": app_bytes / (app_ms * 1e-3) / 1e9,
        "append_bytes": app_bytes,
        "euler_us": float(np.mean(eul)) * 1e3,
        "nq": bt, "nk": nk,
    }
    return res


def gpu_chain_bench(args, Hl, Wl, W, H, d, n_layers, n_stages=4):
    """One block through n_stages timestep-forcing stages on one GPU (la_denoise_chain):
    every stage has its own n_layers rings at its own noise level (1.0, 0.75, ...)."""
    import torch
    import streaming_causal_video_amd as L

    L.lib()
    dev = "cuda"
    bt, st = FRAMES * Hl * Wl, Hl * Wl
    nk = st + (W + 1) * bt
    gen = torch.Generator(device=dev)
    gen.manual_seed(4321)

    def randn(shape, dtype=torch.bfloat16):
        return torch.randn(shape, device=dev, dtype=torch.float32, generator=gen).to(dtype)

    levels = [1.0 + DT * i for i in range(n_stages)]
    log(f"setup: {n_stages} stages x {n_layers} layers, Hl={Hl} Wl={Wl} W={W} H={H} d={d}, "
        f"Nq={bt} Nk={nk}, noise levels {levels}")
    stacks = []
    for i in range(n_stages):
        stack = L.KVRingStack(n_layers, W, bt, st, H, d, torch.bfloat16, levels[i])
        for l in range(n_layers):
            stack.sink_k_raw[l].copy_(randn((st, H, d)))
            stack.sink_v[l].copy_(randn((st, H, d)))
        stacks.append(stack)
    pool = 2  # input blocks shared by the stages (content does not affect timing)
    ins = [[tuple(randn((bt, H, d)) for _ in range(3)) for _ in range(n_layers)] for _ in range(pool)]
    outs = [torch.empty((bt, H, d), dtype=torch.bfloat16, device=dev) for _ in range(n_layers)]
    qws = torch.empty((bt, H, d), dtype=torch.bfloat16, device=dev)
    kws = torch.empty_like(qws)
    sws = torch.empty((st, H, d), dtype=torch.bfloat16, device=dev)
    table = torch.empty(L.la_rope_table_bytes(Hl, Wl, d) // 4, dtype=torch.float32, device=dev)
    L.la_rope_table_fill(table, Hl, Wl, d, THETA)
    lat_shape = (16, 3, 60, 104)
    x = torch.randn(lat_shape, device=dev, generator=gen)
    vels = [torch.randn(lat_shape, device=dev, generator=gen) for _ in range(n_stages)]
    aws = L.AttnWorkspace(bt, H) if args.attn_schedule == "balanced" else None
    torch.cuda.synchronize()
    log(f"allocated {torch.cuda.memory_allocated() / 2**30:.1f} GiB")

    def step(b):
        e = b % pool
        stages = []
        for i in range(n_stages):
            g = dict(rings=stacks[i].states, q_raw=[ins[e][l][0] for l in range(n_layers)],
                     k_raw=[ins[e][l][1] for l in range(n_layers)],
                     v_raw=[ins[e][l][2] for l in range(n_layers)], attn_out=outs,
                     vel=vels[i], dt=DT)
            if b == 1:
                g["sink_k_new"] = [ins[e][l][1][:st] for l in range(n_layers)]
                g["sink_v_new"] = [ins[e][l][2][:st] for l in range(n_layers)]
            stages.append(g)
        L.la_denoise_chain(stages, b, qws, kws, sws, table, Hl, Wl, x=x, frames_per_block=FRAMES,
                           sink_delta=DELTA, theta=THETA, scale=d ** -0.5, attn_ws=aws)

    block = 0
    for _ in range(W + args.warmup):
        block += 1
        step(block)
    torch.cuda.synchronize()
    log(f"warm-up done ({block} blocks)")
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    t0.record()
    for _ in range(args.steps):
        block += 1
        step(block)
    t1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = t0.elapsed_time(t1) / args.steps
    log(f"timed {args.steps} blocks: {ms_step:.3f} ms/block through {n_stages} stages "
        f"(host wall {wall / args.steps * 1e3:.3f} ms/block)")
    return {"ms_per_step": ms_step, "blocks_per_s": 1e3 / ms_step, "nq": bt, "nk": nk,
            "attn_flop_per_block": attn_flops(bt, nk, d, H) * n_layers * n_stages}


# --------------------------------------------------------------------------- oracle on host cores
def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        n = [i.get("num_threads", 0) for i in threadpool_info() if i.get("user_api") == "blas"]
        if n:
            return max(n)
    except Exception:
        pass
    return os.cpu_count() or 1


def cpu_baseline(Hl, Wl, W, H, d, n_layers, budget_s=15.0):
    """Time the float64 oracle on this host on a bounded sample of one step:
    (layer, head) units of RoPE + attention + append, extrapolated to all
    n_layers x H units, plus the Euler update on the whole latent."""
    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    from oracle import Ring, attention_lse, euler_step, rope3d

    rng = np.random.default_rng(0)
    bt, st = FRAMES * Hl * Wl, Hl * Wl
    q = rng.standard_normal((bt, 1, d))
    k = rng.standard_normal((bt, 1, d))
    v = rng.standard_normal((bt, 1, d))
    sk = rng.standard_normal((st, 1, d))
    sv = rng.standard_normal((st, 1, d))
    cached_k = [rng.standard_normal((bt, 1, d)) for _ in range(W)]
    cached_v = [rng.standard_normal((bt, 1, d)) for _ in range(W)]
    f0 = FRAMES * 100
    units = 0
    t_start = time.perf_counter()
    while True:
        ring = Ring(W, NOISE)
        for i in range(W):
            ring.append(i + 1, cached_k[i], cached_v[i], NOISE)
        qr = rope3d(q, FRAMES, Hl, Wl, f0, THETA)
        kr = rope3d(k, FRAMES, Hl, Wl, f0, THETA)
        skr = rope3d(sk, 1, Hl, Wl, f0 + DELTA, THETA)
        ck, cv = ring.keys_values()
        attention_lse(qr, np.concatenate([skr, *ck, kr]), np.concatenate([sv, *cv, v]), d ** -0.5)
        ring.append(W + 1, kr, v, NOISE)
        units += 1
        if time.perf_counter() - t_start >= budget_s or units >= n_layers * H:
            break
    t_units = (time.perf_counter() - t_start) / units
    lat = rng.standard_normal((16, 3, 60, 104)).astype(np.float32)
    vel = rng.standard_normal((16, 3, 60, 104)).astype(np.float32)
    te = time.perf_counter()
    euler_step(lat, vel, DT).astype(np.float32)
    t_euler = time.perf_counter() - te
    t_step = t_units * n_layers * H + t_euler
    return {
        "value": 1.0 / t_step,
        "unit": "blocks/s",
        "cores": blas_threads(),
        "kind": "oracle",
        "sample": (f"{units} of {n_layers * H} (layer, head) units of one step "
                   f"(RoPE of Q, K, sink K + fp64 attention over {bt} x "
                   f"{st + (W + 1) * bt} keys + ring append), timed "
                   f"{t_units * units:.1f} s and scaled x{n_layers * H / units:.0f}; Euler on the "
                   f"whole latent timed once"),
        "seconds_per_step_extrapolated": t_step,
        "host_cpus": os.cpu_count(),
        "host_affinity": len(os.sched_getaffinity(0)),
    }


def gpu_fp8_attn_bench(args, Hl, Wl, W, H, d):
    """e4m3 block attention at the C2 shape (ring full, Nk = sink + (W+1) blocks), timed
    alone: la_block_attn_fwd_fp8 on e4m3 Q/K/V quantised once before the timed region."""
    import torch
    import streaming_causal_video_amd as L

    L.lib()
    dev = "cuda"
    bt, st = FRAMES * Hl * Wl, Hl * Wl
    nk = st + (W + 1) * bt
    gen = torch.Generator(device=dev)
    gen.manual_seed(99)
    sc = 5.0 / 448.0
    inv = float(np.float32(1.0) / np.float32(sc))

    def q8(n):
        x = torch.randn((n, H, d), device=dev, dtype=torch.float32, generator=gen).to(torch.bfloat16)
        out = torch.empty((n, H, d), dtype=torch.uint8, device=dev)
        L.la_quantize_fp8(x, out, inv)
        return out

    ring = L.KVRing(W, bt, st, H, d, torch.uint8, NOISE)
    for b in range(1, W + 1):
        L.la_kvcache_append_evict(ring.state, q8(bt), q8(bt), b, NOISE)
    q, k, v, sk, sv = q8(bt), q8(bt), q8(bt), q8(st), q8(st)
    out = torch.empty((bt, H, d), dtype=torch.bfloat16, device=dev)

    def run():
        L.la_block_attn_fwd_fp8(ring.state, q, sk, sv, k, v, out, sc, sc, sc, scale=d ** -0.5)

    for _ in range(args.warmup + 3):
        run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = []
    for _ in range(5):
        e0.record()
        for _ in range(args.steps):
            run()
        e1.record()
        torch.cuda.synchronize()
        reps.append(e0.elapsed_time(e1) / args.steps)
    ms = sorted(reps)[2]
    fl = attn_flops(bt, nk, d, H)
    log(f"fp8 attention Nq={bt} Nk={nk}: {ms:.3f} ms ({fl / (ms * 1e-3) / 1e12:.1f} TFLOP/s)")
    return {"ms": ms, "tflops": fl / (ms * 1e-3) / 1e12, "flop": fl, "nq": bt, "nk": nk}


def kernel_version(prefix):
    """The library's version tag of one kernel family (e.g. "attn-v9", "fp8-v6")."""
    import streaming_causal_video_amd as L
    return next((t for t in L.la_version().split() if t.startswith(prefix)), None)


def fp8_main(args):
    """--workload c2fp8: the e4m3 attention kernel at the C2 shape."""
    geo = dict(Hl=30, Wl=52, W=4, H=40, d=128)
    r = gpu_fp8_attn_bench(args, **geo)
    version = kernel_version("fp8-")
    out = {
        "metric": "block-attn TFLOP/s at 1 GPU, e4m3 operands; % fp8 MFMA peak",
        "value": round(r["tflops"], 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8-e4m3",
        "data": "synthetic N(0,1) Q/K/V quantised to e4m3 (per-tensor scale 5/448), resident in HBM",
        "config": {"workload": "C2 e4m3 block attention 40x128, Nq 4680, Nk 24960 (W=4 e4m3 ring)",
                   "heads": geo["H"], "head_dim": geo["d"], "nq": r["nq"], "nk": r["nk"]},
        "roofline": {"bound": "mfma", "achieved": round(r["tflops"], 2), "peak": PEAK_FP8_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(r["tflops"] / PEAK_FP8_TFLOPS, 4),
                     "traffic": FP8_TRAFFIC_BYTES.get(version), "kernel": "attn_fp8_kernel",
                     "kernel_version": version, "flop_per_launch": r["flop"]},
    }
    print(json.dumps(out), flush=True)
    return 0


def gpu_refresh_bench(args, Hl, Wl, W, H, d, n_layers, n_steps=4):
    """The clean-cache baseline the pipeline replaces (NFE 5): per block, n_steps denoise
    passes attend to one shared clean cache without writing it (LA_STEP_ATTEND_ONLY), then a
    refresh pass at noise level 0 writes the block's K/V into it."""
    import torch
    import streaming_causal_video_amd as L

    L.lib()
    dev = "cuda"
    bt, st = FRAMES * Hl * Wl, Hl * Wl
    gen = torch.Generator(device=dev)
    gen.manual_seed(777)

    def randn(shape, dtype=torch.bfloat16):
        return torch.randn(shape, device=dev, dtype=torch.float32, generator=gen).to(dtype)

    log(f"setup: clean-cache baseline, {n_layers} layers, {n_steps} attend-only passes + refresh")
    stack = L.KVRingStack(n_layers, W, bt, st, H, d, torch.bfloat16, 0.0)
    for l in range(n_layers):
        stack.sink_k_raw[l].copy_(randn((st, H, d)))
        stack.sink_v[l].copy_(randn((st, H, d)))
    pool = 2
    ins = [[tuple(randn((bt, H, d)) for _ in range(3)) for _ in range(n_layers)] for _ in range(pool)]
    log("inputs ready")
    outs = [torch.empty((bt, H, d), dtype=torch.bfloat16, device=dev) for _ in range(n_layers)]
    qws = torch.empty((bt, H, d), dtype=torch.bfloat16, device=dev)
    kws = torch.empty_like(qws)
    sws = torch.empty((st, H, d), dtype=torch.bfloat16, device=dev)
    table = torch.empty(L.la_rope_table_bytes(Hl, Wl, d) // 4, dtype=torch.float32, device=dev)
    L.la_rope_table_fill(table, Hl, Wl, d, THETA)
    lat_shape = (16, 3, 60, 104)
    x = torch.randn(lat_shape, device=dev, generator=gen)
    vels = [torch.randn(lat_shape, device=dev, generator=gen) for _ in range(n_steps)]
    aws = L.AttnWorkspace(bt, H) if args.attn_schedule == "balanced" else None
    torch.cuda.synchronize()

    def step(b):
        e = b % pool
        q = [ins[e][l][0] for l in range(n_layers)]
        k = [ins[e][l][1] for l in range(n_layers)]
        v = [ins[e][l][2] for l in range(n_layers)]
        for i in range(n_steps):
            L.la_denoise_step(stack.states, b, q, k, v, outs, qws, kws, sws, table, Hl, Wl, FRAMES,
                              DELTA, THETA, scale=d ** -0.5, x=x, vel=vels[i], dt=DT,
                              flags=L.LA_STEP_ATTEND_ONLY, attn_ws=aws)
        L.la_denoise_step(stack.states, b, q, k, v, outs, qws, kws, sws, table, Hl, Wl, FRAMES,
                          DELTA, THETA, scale=d ** -0.5,
                          sink_k_new=[t[:st] for t in k] if b == 1 else None,
                          sink_v_new=[t[:st] for t in v] if b == 1 else None, attn_ws=aws)

    block = 0
    for _ in range(W + args.warmup):
        block += 1
        step(block)
        torch.cuda.synchronize()
        log(f"warm-up block {block} done")
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(args.steps):
        block += 1
        step(block)
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / args.steps
    log(f"clean-cache baseline: {ms:.3f} ms/block ({n_steps} attend-only passes + 1 refresh)")
    return {"ms_per_step": ms, "blocks_per_s": 1e3 / ms}


def refresh_main(args):
    """--workload refresh: blocks/s of the NFE-5 clean-cache baseline on one GPU."""
    geo = dict(Hl=30, Wl=52, W=4, H=40, d=128, n_layers=args.layers or 40)
    r = gpu_refresh_bench(args, **geo)
    out = {
        "metric": "clean-cache baseline blocks/s at 1 GPU (4 attend-only passes + 1 refresh, NFE 5)",
        "value": round(r["blocks_per_s"], 4), "unit": "blocks/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(r["ms_per_step"], 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic N(0,1) Q/K/V, sinks, latent and velocities resident in HBM (no trained weights)",
        "config": {"workload": ("C4 shapes, 40 layers: 4 denoise passes attending to a shared clean "
                                "cache (W=4) + 1 refresh pass writing it, per block"),
                   "layers": geo["n_layers"], "nfe": 5, "parallelism": "none"},
    }
    print(json.dumps(out), flush=True)
    return 0


def chain_main(args):
    """--workload chain: blocks/s of a complete 4-step denoise on one GPU."""
    geo = dict(Hl=30, Wl=52, W=4, H=40, d=128, n_layers=args.layers or 40)
    r = gpu_chain_bench(args, **geo)
    out = {
        "metric": "denoise-chain blocks/s at 1 GPU (4 timestep-forcing stages in sequence)",
        "value": round(r["blocks_per_s"], 4),
        "unit": "blocks/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic N(0,1) Q/K/V, sinks, latent and velocities resident in HBM (no trained weights)",
        "config": {"workload": ("C4 shapes, 4 stages (noise levels 1.0/0.75/0.5/0.25) x 40 layers "
                                "(3D Rolling RoPE + bf16 block attention 40x128, Nq 4680, Nk 24960 "
                                "+ ring append/evict, W=4) + Euler per stage, one GPU"),
                   "stages": 4, "layers": geo["n_layers"], "heads": geo["H"], "head_dim": geo["d"],
                   "block_tokens": r["nq"], "nk": r["nk"],
                   "parallelism": "none (4 stages sequential on 1 GPU)"},
        "attn_tflop_per_block": round(r["attn_flop_per_block"] / 1e12, 3),
    }
    print(json.dumps(out), flush=True)
    return 0


# --------------------------------------------------------------------------- main
def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", choices=["c4", "c2", "c3", "c5", "chain", "c2fp8", "refresh"],
                    default="c4")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--layers", type=int, default=0,
                    help="layers per stage for the chain / refresh workloads (default 40)")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--attn-schedule", choices=["balanced", "grid"], default="balanced",
                    help="attention work schedule: persistent balanced grid with a workspace "
                         "(default) or one workgroup per query tile")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs one GPU's stage only (asked for {args.gpus} GPUs); spreading the "
              "denoise stages over several GPUs is not implemented.", file=sys.stderr)
        return 2
    if int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py is single-process; WORLD_SIZE > 1 is not supported.", file=sys.stderr)
        return 2

    # workloads with their own driver (they take --steps as given)
    if args.workload == "chain":
        return chain_main(args)
    if args.workload == "c2fp8":
        return fp8_main(args)
    if args.workload == "refresh":
        return refresh_main(args)
    if args.workload == "c4":
        geo = dict(Hl=30, Wl=52, W=4, H=40, d=128, n_layers=40)
        name = ("C4 full denoise step: 40 layers x (3D Rolling RoPE + bf16 block attention "
                "40x128, Nq 4680, Nk 24960 + ring append/evict, W=4, 1560-token sink) + "
                "flow-matching Euler on fp32 16x3x60x104")
    elif args.workload == "c2":
        geo = dict(Hl=30, Wl=52, W=4, H=40, d=128, n_layers=1)
        name = "C2 one layer: bf16 block attention 40x128, Nq 4680, Nk 24960 (+RoPE, append, Euler)"
    elif args.workload == "c3":
        geo = dict(Hl=30, Wl=52, W=8, H=40, d=128, n_layers=1)
        name = ("C3 one layer, window of 8 blocks: bf16 block attention 40x128, Nq 4680, "
                "Nk 43680 (+RoPE, append, Euler)")
    elif args.workload == "c5":
        geo = dict(Hl=44, Wl=80, W=4, H=40, d=128, n_layers=1)
        name = ("C5 720p-shaped layer: 44x80 tokens/frame, Nq 10560, Nk 56320 (sink + 4 cached "
                "blocks + block), streamed blocks")
        if args.steps == 10:
            args.steps = 1000
    else:
        raise AssertionError(args.workload)
    r = gpu_step_bench(args, **geo)
    import streaming_causal_video_amd as L
    version = kernel_version("attn-")
    traffic = ATTN_TRAFFIC_BYTES.get(version) if args.workload in ("c4", "c2") else None
    peak_frac = r["attn_tflops"] / PEAK_BF16_TFLOPS
    out = {
        "metric": METRIC,
        "value": round(r["blocks_per_s"], 4),
        "unit": "blocks/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic N(0,1) Q/K/V, sinks, latent and velocity resident in HBM (no trained weights)",
        "config": {"workload": name, "layers": geo["n_layers"], "heads": geo["H"],
                   "head_dim": geo["d"], "block_tokens": r["nq"], "sink_tokens": geo["Hl"] * geo["Wl"],
                   "window_blocks": geo["W"], "nk": r["nk"], "parallelism": "none (1 GPU = 1 stage)"},
        "attn_tflops": round(r["attn_tflops"], 2),
        "attn_ms": round(r["attn_ms"], 4),
        "roofline": {"bound": "mfma", "achieved": round(r["attn_tflops"], 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(peak_frac, 4),
                     "traffic": traffic, "kernel": "attn_bf16_kernel", "kernel_version": version,
                     "flop_per_launch": r["attn_flop_per_launch"]},
        "streaming_kernels": {
            "rope_us": round(r["rope_us"], 2), "rope_GBps": round(r["rope_gbs"], 1),
            "rope_frac_hbm": round(r["rope_gbs"] / PEAK_HBM_GBS, 4),
            "append_us": round(r["append_us"], 2), "append_GBps": round(r["append_gbs"], 1),
            "append_frac_hbm": round(r["append_gbs"] / PEAK_HBM_GBS, 4),
            "euler_us": round(r["euler_us"], 2),
        },
    }
    if not args.no_cpu_baseline:
        log("timing the float64 oracle on host cores ...")
        out["cpu_baseline"] = cpu_baseline(geo["Hl"], geo["Wl"], geo["W"], geo["H"], geo["d"],
                                           geo["n_layers"], args.cpu_budget)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
