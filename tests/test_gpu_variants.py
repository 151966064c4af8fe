"""Cache-semantics variants of the step on the GPU against the float64 oracle (the
pages' ablations: NOTES Table 4 -- no Rolling RoPE, no AAS, a clean cache -- and
the Table 6 finding on a fixed-noise cache)."""

import numpy as np
import pytest

import seeded_inputs as si
from oracle import StreamOracle, euler_step

from gpu_helpers import (FRAMES_PER_BLOCK, SINK_DELTA, THETA, check_attention, to_dev, to_f64,
                         torch)

pytestmark = pytest.mark.gpu

SHAPE = si.SMALL_BF16
N_LAYERS = 2
LAT = (16, 3, 8, 8)


@pytest.fixture(scope="module")
def L():
    import streaming_causal_video_amd as lib
    lib.lib()
    return lib


class Stage:
    """Per-layer rings (with the sinks of the given layer indices) and workspaces."""

    def __init__(self, L, layers, noise):
        t = torch()
        s = SHAPE
        self.layers = layers
        self.stack = L.KVRingStack(len(layers), s.W, s.block_tokens, s.sink_tokens, s.heads,
                                   s.head_dim, t.bfloat16, noise)
        for i, l in enumerate(layers):
            sk, sv = s.initial_sink(l)
            self.stack.sink_k_raw[i].copy_(to_dev(sk))
            self.stack.sink_v[i].copy_(to_dev(sv))


class Work:
    def __init__(self, L):
        t = torch()
        s = SHAPE
        blk = (s.block_tokens, s.heads, s.head_dim)
        self.table = t.empty(L.la_rope_table_bytes(s.Hl, s.Wl, s.head_dim) // 4, dtype=t.float32,
                             device="cuda")
        L.la_rope_table_fill(self.table, s.Hl, s.Wl, s.head_dim, THETA)
        self.qws = t.empty(blk, dtype=t.bfloat16, device="cuda")
        self.kws = t.empty(blk, dtype=t.bfloat16, device="cuda")
        self.sws = t.empty((s.sink_tokens, s.heads, s.head_dim), dtype=t.bfloat16, device="cuda")
        self.outs = [t.empty(blk, dtype=t.bfloat16, device="cuda") for _ in range(N_LAYERS)]
        # attention workspace: the balanced schedule in these passes (None: one
        # workgroup per query tile)
        self.aws = L.AttnWorkspace(s.block_tokens, s.heads)


def run_pass(L, w, rings, layers, b, *, sink_delta=SINK_DELTA, replace_sink=True, flags=0,
             x=None, vel=None):
    """One la_denoise_step over the given per-layer input streams (layer indices)."""
    s = SHAPE
    dev = [tuple(to_dev(z) for z in s.block_inputs(l, b)) for l in layers]
    n = s.sink_tokens
    rep = replace_sink and b == 1 and not flags
    L.la_denoise_step(rings, b, [d[0] for d in dev], [d[1] for d in dev], [d[2] for d in dev],
                      w.outs, w.qws, w.kws, w.sws, w.table, s.Hl, s.Wl, FRAMES_PER_BLOCK,
                      sink_delta, THETA, scale=s.head_dim ** -0.5,
                      sink_k_new=[d[1][:n] for d in dev] if rep else None,
                      sink_v_new=[d[2][:n] for d in dev] if rep else None, x=x, vel=vel,
                      dt=-0.25, flags=flags, attn_ws=w.aws)


def check_outs(w, oracles, b, what):
    torch().cuda.synchronize()
    for i, o in enumerate(oracles):
        check_attention(to_f64(w.outs[i]), o.block_output(b), f"{what} layer {i} block {b}")


@pytest.mark.parametrize("variant", ["no_aas", "no_rolling", "neither"])
def test_rolling_and_aas_ablations(L, variant):
    rolling = variant == "no_aas"
    aas = variant == "no_rolling"
    layers = [0, 1]
    st = Stage(L, layers, 0.75)
    w = Work(L)
    oracles = [StreamOracle(SHAPE, layer=l, rolling=rolling, aas=aas) for l in layers]
    for b in range(1, SHAPE.W + 3):
        # Rolling RoPE off: the sink stays at frame 0, so the offset is -f0(b)
        delta = SINK_DELTA if rolling else -FRAMES_PER_BLOCK * (b - 1)
        run_pass(L, w, st.stack.states, layers, b, sink_delta=delta, replace_sink=aas)
        check_outs(w, oracles, b, variant)
    for r in st.stack.states:
        assert r.sink_replaced == int(aas)


@pytest.mark.parametrize("cache", ["clean_refresh", "fixed_noise"])
def test_shared_cache_baselines(L, cache):
    """clean_refresh: 4 attend-only denoise stages read a clean cache (noise level 0) that a
    fifth pass writes after them (NFE 5).  fixed_noise: stages 1-3 attend only, the stage at
    t = 0.25 writes the one shared cache (all entries at that level)."""
    t = torch()
    stage_layers = [[N_LAYERS * s + l for l in range(N_LAYERS)] for s in range(4)]
    if cache == "clean_refresh":
        writer_layers, writer_noise = [4 * N_LAYERS + l for l in range(N_LAYERS)], 0.0
    else:
        writer_layers, writer_noise = stage_layers[3], 0.25
    shared = Stage(L, writer_layers, writer_noise)
    w = Work(L)
    oracles = [[StreamOracle(SHAPE, layer=l, cache_layer=c) for l, c in zip(ls, writer_layers)]
               for ls in stage_layers]
    writer_orc = [StreamOracle(SHAPE, layer=c) for c in writer_layers]
    lat = si.latent(SHAPE.cfg_id, 0, si.TID_X, LAT)
    x = to_dev(lat)
    x_ref = lat.values.copy()
    for b in range(1, SHAPE.W + 3):
        for s_ in range(4):
            vel = si.latent(SHAPE.cfg_id, 100 * b + s_, si.TID_VEL, LAT)
            writes = cache == "fixed_noise" and s_ == 3
            run_pass(L, w, shared.stack.states, stage_layers[s_], b,
                     flags=0 if writes else L.LA_STEP_ATTEND_ONLY, x=x, vel=to_dev(vel))
            x_ref = euler_step(x_ref, vel.values, -0.25).astype(np.float32).astype(np.float64)
            check_outs(w, writer_orc if writes else oracles[s_], b, f"{cache} stage {s_}")
        if cache == "clean_refresh":
            run_pass(L, w, shared.stack.states, writer_layers, b)  # the refresh pass, no Euler
            check_outs(w, writer_orc, b, "refresh pass")
        np.testing.assert_array_equal(x.cpu().numpy(), x_ref.astype(np.float32))
        for r in shared.stack.states:
            assert r.last_block == b and r.noise_level == np.float32(writer_noise)
    t.cuda.synchronize()
