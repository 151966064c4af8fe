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
ATTN_TRAFFIC_BYTES = {"attn-v9": 8.618e8, "attn-v12": 9.031e8, "attn-v13": 9.128e8, "attn-v14": 9.047e8,
                      "attn-v15": 8.118e8, "attn-v16": 8.916e8, "attn-v17": 8.962e8}
# The same for the e4m3 attention kernel at the C2 shape (--workload c2fp8).
FP8_TRAFFIC_BYTES = {"fp8-v6": 5.337e+08, "fp8-v7": 5.276e+08, "fp8-v8": 5.274e+08,
                     "fp8-v9": 5.338e+08, "fp8-v10": 4.739e+08}


_T0 = time.perf_counter()


def log(msg):
    print(f"[{time.perf_counter() - _T0:7.1f}s] {msg}", file=sys.stderr, flush=True)


def attn_flops(nq, nk, d, h):
    return 4.0 * nq * nk * d * h


# --------------------------------------------------------------------------- GPU
FP8_SCALE = 5.0 / 448.0  # per-tensor e4m3 scale of K and V: |x| = 5 maps to 448


def fp8_factors(d):
    """(dq, dk, dv) of the e4m3 workloads: K and V at 5/448; Q at the least factor >= 5/448
    for which the logit factor scale dq dk log2(e) is a power of two to within 2^-24 (the
    attention's faster path; |q| up to at least 5 still maps into the e4m3 range)."""
    import streaming_causal_video_amd as L
    dq = L.la_fp8_q_factor_pow2(d ** -0.5, FP8_SCALE, FP8_SCALE)
    return dq, FP8_SCALE, FP8_SCALE


def gpu_step_bench(args, Hl, Wl, W, H, d, n_layers, with_euler=True, fp8=False):
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

    staged = args.ring == "staged"
    log(f"setup: {n_layers} layers, Hl={Hl} Wl={Wl} W={W} H={H} d={d}, Nq={bt} Nk={nk}, "
        f"{args.ring} rings")
    stack = L.KVRingStack(n_layers, W, bt, st, H, d, torch.uint8 if fp8 else torch.bfloat16, NOISE,
                          staged=staged)
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
    aws = L.AttnWorkspace(bt, H) if args.attn_schedule == "balanced" and not fp8 else None
    if fp8:
        fdq, fdk, fdv = fp8_factors(d)
        u8 = lambda shp: torch.empty(shp, dtype=torch.uint8, device=dev)
        q8 = u8((bt, H, d))
        k8, v8 = (None, None) if staged else (u8((bt, H, d)), u8((bt, H, d)))
        sk8, sv8 = u8((st, H, d)), u8((st, H, d))
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
        if fp8:
            L.la_denoise_step_fp8(stack.states, b, q, k, v, outs, None, None, None, q8, k8, v8, sk8,
                                  sv8, table, Hl, Wl, FRAMES, DELTA, THETA, scale=d ** -0.5,
                                  dq=fdq, dk=fdk, dv=fdv, sink_k_new=skn,
                                  sink_v_new=svn, x=x, vel=vels[e] if with_euler else None,
                                  dt=DT, timing_events=events)
            return
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
        if staged:
            # a staged ring's append launches nothing (the RoPE launch staged K and V):
            # its span is not taken, which keeps two event packets per layer off the stream
            for l in range(n_layers):
                arr[6 * l + 4] = arr[6 * l + 5] = None
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
    app_ms = 0.0 if staged else avg(4)[0]
    # per timed block: attention time of each layer's launch, averaged over the layers
    per_block = [float(np.mean([objs[6 * l + 2].elapsed_time(objs[6 * l + 3])
                                for l in range(n_layers)])) for objs in ev_objs]
    per_block_step = [objs[0].elapsed_time(objs[6 * n_layers + 1]) for objs in ev_objs]
    eul = [objs[6 * n_layers].elapsed_time(objs[6 * n_layers + 1]) for objs in ev_objs]
    log(f"timed {args.steps} steps: {ms_step:.3f} ms/step (host wall {wall / args.steps * 1e3:.3f} ms/step)")
    fl = attn_flops(bt, nk, d, H)
    # the bf16 step's RoPE launch rotates K and the sink K and writes the block tokens'
    # float32 cos/sin for Q (d * 4 bytes a token; the attention kernel rotates Q as it
    # loads it); the e4m3 step's rotates Q as well
    rope_bytes = (2 * ((2 * bt if fp8 else bt) + st) * H * d * 2) + (0 if fp8 else bt * d * 4)
    # plain rings: the append copies K and V after the attention; staged rings: the
    # RoPE launch also writes K into the next slot and copies V there, so the append
    # only records the block
    app_bytes = 0 if staged else 2 * 2 * bt * H * d * 2
    if staged and not fp8:
        rope_bytes += 2 * bt * H * d * 2
    if fp8:
        # one launch rotates Q, K and the sink K and quantises them with V and the sink V
        # (bf16 in, e4m3 out); a staged e4m3 ring takes the K and V codes in place, so the
        # append copies nothing
        rope_bytes = (3 * bt + 2 * st) * H * d * 3
        app_bytes = 0 if staged else 2 * 2 * bt * H * d
    res = {
        "ms_per_step": ms_step,
        "blocks_per_s": 1e3 / ms_step,
        "attn_ms": attn_ms, "attn_ms_sd": attn_sd,
        "attn_tflops": fl / (attn_ms * 1e-3) / 1e12,
        "attn_flop_per_launch": fl,
        "rope_us": rope_ms * 1e3, "rope_gbs": rope_bytes / (rope_ms * 1e-3) / 1e9,
        "rope_bytes": rope_bytes,
        "append_us": app_ms * 1e3,
        "append_gbs": app_bytes / (app_ms * 1e-3) / 1e9 if app_bytes else 0.0,
        "append_bytes": app_bytes,
        "euler_us": float(np.mean(eul)) * 1e3,
        "nq": bt, "nk": nk,
        "first_block": block - args.steps + 1,
        "per_block_attn_ms": per_block, "per_block_step_ms": per_block_step,
    }
    return res


def drift(first_block, per_block):
    """Drift of a per-block series: means of the first and last tenth and the slope of a
    least-squares line, in % of the mean per 100 blocks."""
    y = np.asarray(per_block)
    n = len(y)
    k = max(1, n // 10)
    x = np.arange(first_block, first_block + n)
    slope = float(np.polyfit(x, y, 1)[0]) if n > 1 else 0.0
    return {"blocks": f"{first_block}-{first_block + n - 1}", "mean_ms": round(float(y.mean()), 4),
            "first_tenth_ms": round(float(y[:k].mean()), 4),
            "last_tenth_ms": round(float(y[-k:].mean()), 4),
            "slope_pct_per_100_blocks": round(100 * 100 * slope / float(y.mean()), 3),
            "cv_pct": round(100 * float(y.std() / y.mean()), 2)}


def hbm_kernels_bench(Hl, Wl, W, H, d, reps=24, euler_elems=1 << 28):
    """The HBM-bound kernels alone, each launched `reps` times back to back between two
    events over rotating buffers whose total exceeds the 256 MB last-level cache (so
    every launch streams from HBM): RoPE of Q, K and the sink K (six input and six
    output sets), the ring append (six K/V input sets into a 4-slot ring), and the
    Euler update of a batched latent of `euler_elems` float32 values (x and v 1 GiB
    each at the default).  RoPE and the append are checked once through the Python
    binding and then called through the C entry points with their arguments built
    beforehand, so that the host's marshalling does not pace the launches.  Returns
    per-launch microseconds and GB/s."""
    import ctypes

    import torch
    import streaming_causal_video_amd as L
    from streaming_causal_video_amd._lib import LA_OK

    dev = "cuda"
    bt, st = FRAMES * Hl * Wl, Hl * Wl
    gen = torch.Generator(device=dev)
    gen.manual_seed(55)

    def randn(shape, dtype=torch.bfloat16):
        return torch.randn(shape, device=dev, dtype=torch.float32, generator=gen).to(dtype)

    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed(fn, n=reps):
        fn(0)
        torch.cuda.synchronize()
        e0.record()
        for i in range(n):
            fn(i)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n * 1e3  # us per launch

    res = {}
    nsets = 6
    table = torch.empty(L.la_rope_table_bytes(Hl, Wl, d) // 4, dtype=torch.float32, device=dev)
    L.la_rope_table_fill(table, Hl, Wl, d, THETA)
    ins = [(randn((bt, H, d)), randn((bt, H, d)), randn((st, H, d))) for _ in range(nsets)]
    outs = [tuple(torch.empty_like(t) for t in s) for s in ins]

    lib = L.lib()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    ptr = lambda t: ctypes.c_void_p(t.data_ptr())
    qs = float(np.float32(d ** -0.5 * np.log2(np.e)))
    statuses = []
    rope_args = []
    # the whole la_rope3d_rolling call (Q, K and the sink K): 224 MB at C2, about the
    # bytes of the step's fused launch (K, the sink K, Q's cos/sin and the V staging)
    for j in range(nsets):
        a, b = ins[j], outs[j]
        L.la_rope3d_rolling(a[0], b[0], a[1], b[1], FRAMES, 300 + 3 * j, a[2], b[2], DELTA, table,
                            Hl, Wl, H, d, THETA, q_scale=qs)
        rope_args.append((ptr(a[0]), ptr(b[0]), ptr(a[1]), ptr(b[1]), FRAMES, 300 + 3 * j,
                          ptr(a[2]), ptr(b[2]), DELTA, ptr(table), Hl, Wl, H, d, L.LA_BF16, THETA,
                          qs, stream))

    def rope(i):
        statuses.append(lib.la_rope3d_rolling(*rope_args[i % nsets]))

    rope_bytes = 2 * (2 * bt + st) * H * d * 2
    us = timed(rope)
    res.update(rope_us=us, rope_GBps=rope_bytes / (us * 1e-6) / 1e9)
    del outs
    ring = L.KVRing(W, bt, st, H, d, torch.bfloat16, NOISE)
    L.la_kvcache_append_evict(ring.state, ins[0][0], ins[0][1], 1, NOISE)
    block = [1]
    evicted = ctypes.c_int64()
    app_args = [(ptr(ins[j][0]), ptr(ins[j][1])) for j in range(nsets)]

    def append(i):
        block[0] += 1
        statuses.append(lib.la_kvcache_append_evict(ctypes.byref(ring.state), *app_args[i % nsets],
                                                    block[0], NOISE, ctypes.byref(evicted),
                                                    stream))

    app_bytes = 2 * 2 * bt * H * d * 2
    us = timed(append)
    res.update(append_us=us, append_GBps=app_bytes / (us * 1e-6) / 1e9)
    if any(st_ != LA_OK for st_ in statuses):
        raise RuntimeError(f"standalone launches failed: {sorted(set(statuses))}")
    del ring, ins
    torch.cuda.empty_cache()
    x = torch.randn(euler_elems, device=dev, generator=gen)
    v = torch.randn(euler_elems, device=dev, generator=gen)
    eul_reps = 8

    def euler(i):
        L.la_fm_euler_step(x, v, DT)

    e_bytes = 3 * 4 * euler_elems
    us = timed(euler, eul_reps)
    res.update(euler_batched_elems=euler_elems, euler_batched_us=us,
               euler_batched_GBps=e_bytes / (us * 1e-6) / 1e9)
    del x, v
    torch.cuda.empty_cache()
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
        stack = L.KVRingStack(n_layers, W, bt, st, H, d, torch.bfloat16, levels[i],
                              staged=args.ring == "staged")
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


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(Hl, Wl, W, H, d, n_layers, budget_s=15.0):
    """Time the float64 oracle on this host, part by part, at the workload's sizes, in
    the GPU's units: RoPE of the whole block's Q and K and of the sink K (GB/s of the
    kernel's bf16 bytes), the ring append of a whole block (GB/s), the Euler update of
    the 16x3x60x104 latent (GB/s), and attention over all Nk keys for as many heads as
    fit in `budget_s` (TFLOP/s); the step's time is then extrapolated to all heads and
    layers (stated in `sample`)."""
    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    from oracle import Ring, attention_lse, euler_step, rope3d

    rng = np.random.default_rng(0)
    bt, st = FRAMES * Hl * Wl, Hl * Wl
    nk = st + (W + 1) * bt
    f0 = FRAMES * 100

    def clock(fn):
        t = time.perf_counter()
        out = fn()
        return time.perf_counter() - t, out

    q = rng.standard_normal((bt, H, d))
    k = rng.standard_normal((bt, H, d))
    v = rng.standard_normal((bt, H, d))
    sk = rng.standard_normal((st, H, d))
    sv = rng.standard_normal((st, H, d))
    t_rope, (qr, kr, skr) = clock(lambda: (rope3d(q, FRAMES, Hl, Wl, f0, THETA),
                                           rope3d(k, FRAMES, Hl, Wl, f0, THETA),
                                           rope3d(sk, 1, Hl, Wl, f0 + DELTA, THETA)))
    ring = Ring(W, NOISE)
    for i in range(W):
        ring.append(i + 1, rng.standard_normal((bt, H, d)), rng.standard_normal((bt, H, d)),
                    NOISE)
    ck, cv = ring.keys_values()
    keys = np.concatenate([skr, *ck, kr])
    vals = np.concatenate([sv, *cv, v])
    t_att, heads_done = 0.0, 0
    while heads_done < H and (heads_done == 0 or t_att < budget_s):
        h = heads_done
        dt_h, _ = clock(lambda: attention_lse(qr[:, h:h + 1], keys[:, h:h + 1], vals[:, h:h + 1],
                                              d ** -0.5))
        t_att += dt_h
        heads_done += 1
    t_head = t_att / heads_done
    t_app, _ = clock(lambda: ring.append(W + 1, kr, v, NOISE))
    lat = rng.standard_normal((16, 3, 60, 104)).astype(np.float32)
    vel = rng.standard_normal((16, 3, 60, 104)).astype(np.float32)
    t_eul, _ = clock(lambda: euler_step(lat, vel, DT).astype(np.float32))
    t_layer = t_rope + H * t_head + t_app
    t_step = n_layers * t_layer + t_eul
    rope_bytes = 2 * (2 * bt + st) * H * d * 2
    app_bytes = 2 * 2 * bt * H * d * 2
    flop_head = 4.0 * bt * nk * d
    try:
        from threadpoolctl import threadpool_info
        blas = [(i.get("internal_api"), i.get("num_threads")) for i in threadpool_info()
                if i.get("user_api") == "blas"]
    except Exception:
        blas = []
    return {
        "value": 1.0 / t_step,
        "unit": "blocks/s",
        "cores": blas_threads(),
        "kind": "oracle",
        "sample": (f"float64 numpy oracle at {bt} queries x {nk} keys x {H} heads x {d}: RoPE of "
                   f"the whole Q, K and sink K and the ring append of a whole block timed once, "
                   f"attention timed on {heads_done} of {H} heads ({t_att:.1f} s) and scaled "
                   f"x{H / heads_done:.0f}, then x{n_layers} layers, plus the Euler update of "
                   f"the 16x3x60x104 latent"),
        "seconds_per_step_extrapolated": t_step,
        "cpu_model": cpu_model(),
        "host_cpus": os.cpu_count(),
        "host_affinity": len(os.sched_getaffinity(0)),
        "blas": [f"{api}:{n}" for api, n in blas],
        "attn_tflops": flop_head / t_head / 1e12,
        "rope_GBps": rope_bytes / t_rope / 1e9,
        "append_GBps": app_bytes / t_app / 1e9,
        "euler_GBps": 3 * 4 * lat.size / t_eul / 1e9,
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
    dq, dk, dv = fp8_factors(d)

    def q8(n, f):
        x = torch.randn((n, H, d), device=dev, dtype=torch.float32, generator=gen).to(torch.bfloat16)
        out = torch.empty((n, H, d), dtype=torch.uint8, device=dev)
        L.la_quantize_fp8(x, out, float(np.float32(1.0) / np.float32(f)))
        return out

    ring = L.KVRing(W, bt, st, H, d, torch.uint8, NOISE)
    for b in range(1, W + 1):
        L.la_kvcache_append_evict(ring.state, q8(bt, dk), q8(bt, dv), b, NOISE)
    q, k, v, sk, sv = q8(bt, dq), q8(bt, dk), q8(bt, dv), q8(st, dk), q8(st, dv)
    out = torch.empty((bt, H, d), dtype=torch.bfloat16, device=dev)

    def run():
        L.la_block_attn_fwd_fp8(ring.state, q, sk, sv, k, v, out, dq, dk, dv, scale=d ** -0.5)

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
        "data": ("synthetic N(0,1) Q/K/V quantised to e4m3 (per-tensor factors: K, V 5/448, Q the "
                 "least >= 5/448 with a power-of-two logit factor), resident in HBM"),
        "config": {"workload": "C2 e4m3 block attention 40x128, Nq 4680, Nk 24960 (W=4 e4m3 ring)",
                   "heads": geo["H"], "head_dim": geo["d"], "nq": r["nq"], "nk": r["nk"]},
        "roofline": {"bound": "mfma", "achieved": round(r["tflops"], 2), "peak": PEAK_FP8_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(r["tflops"] / PEAK_FP8_TFLOPS, 4),
                     "traffic": FP8_TRAFFIC_BYTES.get(version), "kernel": "attn_fp8_kernel",
                     "kernel_version": version, "flop_per_launch": r["flop"]},
    }
    print(json.dumps(out), flush=True)
    return 0


def c4fp8_main(args):
    """--workload c4fp8: the C4 step on e4m3 rings (la_denoise_step_fp8): one launch of
    RoPE and quantisation, e4m3 attention, the append of K/V codes, Euler."""
    geo = dict(Hl=30, Wl=52, W=4, H=40, d=128, n_layers=40)
    r = gpu_step_bench(args, fp8=True, **geo)
    version = kernel_version("fp8-")
    tf = r["attn_tflops"]
    out = {
        "metric": "denoise-step blocks/s at 1 GPU with e4m3 attention; % fp8 MFMA peak",
        "value": round(r["blocks_per_s"], 4),
        "unit": "blocks/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8-e4m3",
        "data": ("synthetic N(0,1) Q/K/V (bf16), sinks, latent and velocity resident in HBM; "
                 "Q, K, V quantised to e4m3 with per-tensor factors (K, V 5/448, Q the least "
                 ">= 5/448 with a power-of-two logit factor)"),
        "config": {"workload": ("C4 denoise step on e4m3 rings: 40 layers x (3D Rolling RoPE + "
                                "e4m3 quantisation + e4m3 block attention 40x128, Nq 4680, Nk "
                                "24960 + ring append/evict, W=4) + Euler on fp32 16x3x60x104"),
                   "layers": 40, "heads": 40, "head_dim": 128, "block_tokens": r["nq"],
                   "nk": r["nk"], "rings": args.ring,
                   "parallelism": "none (1 GPU = 1 stage)"},
        "attn_tflops": round(tf, 2),
        "attn_ms": round(r["attn_ms"], 4),
        "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_FP8_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tf / PEAK_FP8_TFLOPS, 4),
                     # the same launch shape as --workload c2fp8's, where the counters were read
                     "traffic": FP8_TRAFFIC_BYTES.get(version), "kernel": "attn_fp8_kernel",
                     "kernel_version": version,
                     "flop_per_launch": r["attn_flop_per_launch"]},
        "streaming_kernels": {
            "method": ("in the step: each kernel's own begin and end timestamps (HIP events "
                       "given to its launch), mean over layers and timed steps"),
            "rope_and_quantise_us": round(r["rope_us"], 2),
            "rope_and_quantise_GBps": round(r["rope_gbs"], 1),
            "append_us": round(r["append_us"], 2), "append_bytes": r["append_bytes"],
            "euler_us": round(r["euler_us"], 2),
        },
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
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default: 20 for c4, c2 and c4fp8; 192 for c3, blocks "
                         "9-200; 1000 for c5; 10 for the other workloads)")
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed steps after the ring has filled (default 20; 0 for c3).  "
                         "After a cold start the first blocks run up to 4 %% slower while the "
                         "clock settles, and six warm-up steps left the first timed one 3.7 %% "
                         "slower than the last")
    ap.add_argument("--workload", choices=["c4", "c2", "c3", "c5", "chain", "c2fp8", "c4fp8",
                                           "refresh"],
                    default="c4")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--layers", type=int, default=0,
                    help="layers per stage for the chain / refresh workloads (default 40)")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--ring", choices=["staged", "plain"], default="staged",
                    help="staged: W + 1 slots per ring, the RoPE launch writes K into the next "
                         "slot and copies V there, the append only records the block (fused); "
                         "plain: W slots, the append copies K and V")
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

    default_steps = {"c4": 20, "c2": 20, "c4fp8": 20, "c3": 192, "c5": 1000}
    if args.steps is None:
        args.steps = default_steps.get(args.workload, 10)
    if args.warmup is None:
        args.warmup = 0 if args.workload == "c3" else 20

    # workloads with their own driver (they take --steps as given)
    if args.workload == "chain":
        return chain_main(args)
    if args.workload == "c2fp8":
        return fp8_main(args)
    if args.workload == "refresh":
        return refresh_main(args)
    if args.workload == "c4fp8":
        return c4fp8_main(args)
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
        name = ("C3 one layer, window of 8 blocks, 200 streamed blocks: bf16 block attention "
                "40x128, Nq 4680, Nk 43680 (+RoPE, append, Euler)")
        # by default blocks 1..8 fill the ring and blocks 9..200 are timed
    elif args.workload == "c5":
        geo = dict(Hl=44, Wl=80, W=4, H=40, d=128, n_layers=1)
        name = ("C5 720p-shaped layer: 44x80 tokens/frame, Nq 10560, Nk 56320 (sink + 4 cached "
                "blocks + block), streamed blocks")
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
                   "window_blocks": geo["W"], "nk": r["nk"],
                   "rings": ("staged: W + 1 slots; the RoPE launch writes the rotated K into "
                             "the next slot and copies V there, the append only records the "
                             "block (fused)" if args.ring == "staged" else
                             "plain: W slots, the append copies K and V"),
                   "parallelism": "none (1 GPU = 1 stage)"},
        "attn_tflops": round(r["attn_tflops"], 2),
        "attn_ms": round(r["attn_ms"], 4),
        "per_block_drift": {"attention": drift(r["first_block"], r["per_block_attn_ms"]),
                            "step": drift(r["first_block"], r["per_block_step_ms"])},
        "roofline": {"bound": "mfma", "achieved": round(r["attn_tflops"], 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(peak_frac, 4),
                     "traffic": traffic, "kernel": "attn_bf16_kernel", "kernel_version": version,
                     "flop_per_launch": r["attn_flop_per_launch"]},
        "streaming_kernels": {
            "method": ("in the step: each kernel's own begin and end timestamps (HIP events "
                       "given to its launch), mean over layers and timed steps"),
            "rope_us": round(r["rope_us"], 2), "rope_GBps": round(r["rope_gbs"], 1),
            "rope_frac_hbm": round(r["rope_gbs"] / PEAK_HBM_GBS, 4),
            "rope_bytes": r["rope_bytes"],
            "rope_launch": ("K and the sink K rotated, the block tokens' cos/sin for Q (the "
                            "attention rotates Q), and the block's V copied into the ring's "
                            "next slot (the append's copy)" if args.ring == "staged" else
                            "K and the sink K rotated, the block tokens' cos/sin for Q"),
            "append_us": round(r["append_us"], 2) if r["append_bytes"] else None,
            "append_GBps": round(r["append_gbs"], 1) if r["append_bytes"] else None,
            "append_frac_hbm": (round(r["append_gbs"] / PEAK_HBM_GBS, 4)
                                if r["append_bytes"] else None),
            "append_bytes": r["append_bytes"],
            "euler_us": round(r["euler_us"], 2),
        },
    }
    if args.workload in ("c4", "c2", "c5"):
        hb = hbm_kernels_bench(geo["Hl"], geo["Wl"], geo["W"], geo["H"], geo["d"])
        sk = out["streaming_kernels"]
        sk["standalone"] = {
            "method": ("each kernel launched 24 times back to back between two HIP events over "
                       "rotating buffers larger than the 256 MB last-level cache (Euler: 8 "
                       "launches on a batched latent); per-launch average"),
            "rope_us": round(hb["rope_us"], 2), "rope_GBps": round(hb["rope_GBps"], 1),
            "rope_frac_hbm": round(hb["rope_GBps"] / PEAK_HBM_GBS, 4),
            "append_us": round(hb["append_us"], 2), "append_GBps": round(hb["append_GBps"], 1),
            "append_frac_hbm": round(hb["append_GBps"] / PEAK_HBM_GBS, 4),
            "euler_batched_elems": hb["euler_batched_elems"],
            "euler_batched_us": round(hb["euler_batched_us"], 1),
            "euler_batched_GBps": round(hb["euler_batched_GBps"], 1),
            "euler_batched_frac_hbm": round(hb["euler_batched_GBps"] / PEAK_HBM_GBS, 4),
        }
        log(f"standalone HBM kernels: RoPE {hb['rope_GBps']:.0f} GB/s, append "
            f"{hb['append_GBps']:.0f} GB/s, batched Euler {hb['euler_batched_GBps']:.0f} GB/s")
    if not args.no_cpu_baseline:
        log("timing the float64 oracle on host cores ...")
        out["cpu_baseline"] = cpu_baseline(geo["Hl"], geo["Wl"], geo["W"], geo["H"], geo["d"],
                                           geo["n_layers"], args.cpu_budget)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
