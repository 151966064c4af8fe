"""GPU parity of block attention over {sink, rolling cache, block}, streamed through
the C ABI (RoPE -> attention -> append, sink replaced after block 1), against the
float64 oracle run on the same seeded raw inputs with its own RoPE."""

import numpy as np
import pytest

import seeded_inputs as si
from oracle import StreamOracle, attention_lse

from gpu_helpers import (F32_MAX_ABS, GpuLayerStream, check_attention, say, to_dev, to_f64,
                         torch)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def L():
    import streaming_causal_video_amd as lib
    lib.lib()
    return lib


def _compare_block(gs, orc, b, rows=None, heads=None, lse_tol=None):
    t = torch()
    t.cuda.synchronize()
    got = to_f64(gs.out)
    ref, lse_ref = orc.block_output(b, rows=rows, with_lse=True)
    hs = orc.heads
    g = got[:, hs, :] if rows is None else got[rows][:, hs, :]
    what = f"cfg {gs.shape.cfg_id} block {b}"
    if gs.shape.dtype == "f32":
        err = np.abs(g - ref).max()
        assert err <= F32_MAX_ABS, f"{what}: max-abs {err:.3e}"
    else:
        check_attention(g, ref, what)
    if lse_tol is not None and gs.lse is not None:
        gl = gs.lse.cpu().numpy().astype(np.float64)[hs]
        gl = gl if rows is None else gl[:, rows]
        assert np.abs(gl - lse_ref).max() <= lse_tol, f"{what}: lse"


@pytest.mark.parametrize("shape,nblocks", [
    (si.C1, 10),                # fp32, 10 streamed blocks, AAS after block 1
    (si.SMALL_F32, 6),
    (si.SMALL_F32_D128, 5),
    (si.SMALL_BF16, 6),         # ragged: 35-token frames, 105-token blocks
    (si.MID_BF16, 6),           # several query tiles and key tiles
])
def test_stream_every_block_full_output(L, shape, nblocks):
    say(f"stream cfg {shape.cfg_id} x{nblocks}")
    gs = GpuLayerStream(shape, keep_lse=True)
    orc = StreamOracle(shape)
    lse_tol = 1e-5 if shape.dtype == "f32" else 5e-3
    for b in range(1, nblocks + 1):
        gs.step(b)
        _compare_block(gs, orc, b, lse_tol=lse_tol)


def test_window_of_one_block(L):
    shape = si.LayerShape(105, "bf16", heads=2, head_dim=128, Hl=6, Wl=11, W=1)
    gs = GpuLayerStream(shape)
    orc = StreamOracle(shape)
    for b in range(1, 5):
        gs.step(b)
        _compare_block(gs, orc, b)


def _rows(n, seed, k=96):
    rng = np.random.default_rng(seed)
    r = np.unique(np.concatenate([[0, 1, 63, 64, 127, 128, n - 1], rng.integers(0, n, size=k)]))
    return r[r < n]


@pytest.mark.parametrize("shape", [si.C2, si.C2_PRESCALED])
def test_c2_full_size_sampled(L, shape):
    """One 40x128 layer at 480x832: blocks 1..5 streamed, block 1 (Nk 6240) and block 5
    (Nk 24960) checked on sampled rows of three heads."""
    say(f"C2 full size cfg {shape.cfg_id}")
    gs = GpuLayerStream(shape, keep_lse=True)
    orc = StreamOracle(shape, heads=[0, 21, 39])
    rows = _rows(shape.block_tokens, 5)
    for b in range(1, 6):
        gs.step(b)
        if b in (1, 5):
            _compare_block(gs, orc, b, rows=rows, lse_tol=5e-3)


def test_c5_full_size_sampled(L):
    """720p-shaped layer: Nk = 3520 + 4*10560 + 10560 = 56320 at block 5, with eviction at 6."""
    shape = si.C5
    say("C5 full size")
    gs = GpuLayerStream(shape)
    orc = StreamOracle(shape, heads=[3, 38])
    rows = _rows(shape.block_tokens, 6, k=48)
    for b in range(1, 7):
        gs.step(b)
        if b in (5, 6):
            _compare_block(gs, orc, b, rows=rows)


def test_determinism(L):
    """Two attention calls on an unchanged ring give identical bits."""
    t = torch()
    gs = GpuLayerStream(si.MID_BF16)
    for b in range(1, 5):
        gs.step(b)
    v5 = gs.block_dev(5)[2]
    L.la_block_attn_fwd(gs.ring.state, gs.q_rot, gs.sink_k_rot, gs.k_rot, v5, gs.out)
    first = gs.out.clone()
    L.la_block_attn_fwd(gs.ring.state, gs.q_rot, gs.sink_k_rot, gs.k_rot, v5, gs.out)
    t.cuda.synchronize()
    assert t.equal(first.view(t.int16), gs.out.view(t.int16))


def test_peaked_logits_on_given_bf16_inputs(L):
    """Attention alone on bf16 Q/K/V that the oracle defines, with Q and K scaled by 4
    (logit std ~16, V stays N(0,1)): the row max moves between tiles and segments.
    Both sides read the same bf16 values (x4 is exact in bf16)."""
    t = torch()
    s = si.LayerShape(106, "bf16", heads=3, head_dim=128, Hl=10, Wl=13, W=2)
    x4 = lambda st: si.make_stored(st.values * 4.0, "bf16")
    ring = L.KVRing(s.W, s.block_tokens, s.sink_tokens, s.heads, s.head_dim, t.bfloat16, 0.75)
    keys, vals = [], []
    sk, sv = s.initial_sink(0)
    sk = x4(sk)
    ring.sink_k_raw.copy_(to_dev(sk))
    ring.sink_v.copy_(to_dev(sv))
    for b in range(1, 3):
        _, k, v = s.block_inputs(0, b)
        k = x4(k)
        L.la_kvcache_append_evict(ring.state, to_dev(k), to_dev(v), b, 0.75)
        keys.append(k.values)
        vals.append(v.values)
    q, kc, vc = s.block_inputs(0, 3)
    q, kc = x4(q), x4(kc)
    out = t.empty((s.block_tokens, s.heads, s.head_dim), dtype=t.bfloat16, device="cuda")
    L.la_block_attn_fwd(ring.state, to_dev(q), ring.sink_k_raw, to_dev(kc), to_dev(vc), out)
    t.cuda.synchronize()
    allk = np.concatenate([sk.values, *keys, kc.values])
    allv = np.concatenate([sv.values, *vals, vc.values])
    ref, _ = attention_lse(q.values, allk, allv, s.head_dim ** -0.5)
    check_attention(to_f64(out), ref, "peaked")


def test_late_dominant_keys_raise_the_reference(L):
    """Attention alone on given bf16 inputs where, late in the block's own keys, key
    p_i is a multiple of query i chosen so that query i's logit there is ~100 binades
    above every earlier one: the kernel must raise its running reference mid-stream
    (probabilities against a stale reference would overflow) and rescale what it has
    accumulated.  Query i's output is then essentially V[p_i]; the oracle decides."""
    t = torch()
    s = si.LayerShape(109, "bf16", heads=3, head_dim=128, Hl=10, Wl=13, W=2)
    ring = L.KVRing(s.W, s.block_tokens, s.sink_tokens, s.heads, s.head_dim, t.bfloat16, 0.75)
    keys, vals = [], []
    sk, sv = s.initial_sink(0)
    ring.sink_k_raw.copy_(to_dev(sk))
    ring.sink_v.copy_(to_dev(sv))
    for b in range(1, 3):
        _, k, v = s.block_inputs(0, b)
        L.la_kvcache_append_evict(ring.state, to_dev(k), to_dev(v), b, 0.75)
        keys.append(k.values)
        vals.append(v.values)
    q, kc, vc = s.block_inputs(0, 3)
    kv = kc.values.copy()
    planted = {0: 389, 47: 300, 48: 230, 191: 150, 192: 260, 389: 388}  # query row -> key row
    d = s.head_dim
    for i, p in planted.items():
        for h in range(s.heads):
            qi = q.values[i, h]
            alpha = 100.0 * np.sqrt(d) / (np.log2(np.e) * float(qi @ qi))
            kv[p, h] = alpha * qi
    kc = si.make_stored(kv, "bf16")
    out = t.empty((s.block_tokens, s.heads, s.head_dim), dtype=t.bfloat16, device="cuda")
    lse = t.empty((s.heads, s.block_tokens), dtype=t.float32, device="cuda")
    L.la_block_attn_fwd(ring.state, to_dev(q), ring.sink_k_raw, to_dev(kc), to_dev(vc), out, lse)
    t.cuda.synchronize()
    allk = np.concatenate([sk.values, *keys, kc.values])
    allv = np.concatenate([sv.values, *vals, vc.values])
    ref, lse_ref = attention_lse(q.values, allk, allv, d ** -0.5)
    got = to_f64(out)
    check_attention(got, ref, "late dominant keys")
    rows = sorted(planted)
    assert np.abs(got[rows] - vc.values[[planted[i] for i in rows]]).max() <= 2e-2
    gl = lse.cpu().numpy().astype(np.float64)
    assert np.abs(gl - lse_ref).max() <= 5e-3


@pytest.mark.parametrize("sink,block", [(2, 5), (1, 1), (3, 40)])
def test_tiny_key_ranges(L, sink, block):
    """First block of a ring with no cached blocks: only sink + block keys (as few
    as 2), so the first 64-key tile is also the last and most of it is masked."""
    t = torch()
    heads, d = 2, 128
    cfg = 1100 + 100 * sink + block
    bf = lambda tid, n: si.tensor(cfg, 0, 1, tid, (n, heads, d), "bf16")
    q, kc, vc = bf(si.TID_Q, block), bf(si.TID_K, block), bf(si.TID_V, block)
    sk, sv = bf(si.TID_SINK_K, sink), bf(si.TID_SINK_V, sink)
    ring = L.KVRing(1, block, sink, heads, d, t.bfloat16, 0.75)
    ring.sink_k_raw.copy_(to_dev(sk))
    ring.sink_v.copy_(to_dev(sv))
    out = t.empty((block, heads, d), dtype=t.bfloat16, device="cuda")
    lse = t.empty((heads, block), dtype=t.float32, device="cuda")
    L.la_block_attn_fwd(ring.state, to_dev(q), ring.sink_k_raw, to_dev(kc), to_dev(vc), out, lse)
    t.cuda.synchronize()
    ref, lse_ref = attention_lse(q.values, np.concatenate([sk.values, kc.values]),
                                 np.concatenate([sv.values, vc.values]), d ** -0.5)
    check_attention(to_f64(out), ref, f"sink {sink} block {block}")
    assert np.abs(lse.cpu().numpy().astype(np.float64) - lse_ref).max() <= 5e-3
