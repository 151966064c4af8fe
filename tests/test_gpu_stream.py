"""Long streams and the whole-stage step driver on the GPU, against the float64 oracle."""

import ctypes

import numpy as np
import pytest

import seeded_inputs as si
from oracle import StreamOracle, euler_step

from gpu_helpers import (FRAMES_PER_BLOCK, NOISE_LEVEL, SINK_DELTA, THETA, GpuLayerStream,
                         check_attention, oracle_block_all_heads, rel_l2, say, softmax_scale,
                         to_dev, to_f64, torch)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def L():
    import streaming_causal_video_amd as lib
    lib.lib()
    return lib


@pytest.mark.timeout(900)
def test_c3_200_blocks_checked_at_1_50_200(L):
    """40x128 layer, window 8 (Nk 43680 in steady state), 200 streamed blocks with
    Rolling-RoPE re-offset, append/evict and the sink replacement after block 1; blocks
    1, 50 and 200 compared with the oracle on sampled rows of all 40 heads."""
    t = torch()
    shape = si.C3
    gs = GpuLayerStream(shape)
    rng = np.random.default_rng(7)
    rows = np.unique(np.concatenate([[0, 4679], rng.integers(0, shape.block_tokens, 64)]))
    for b in range(1, 201):
        gs.step(b)
        if b in (1, 50, 200):
            t.cuda.synchronize()
            got = to_f64(gs.out)[rows]
            ref, _ = oracle_block_all_heads(shape, b, rows=rows)
            check_attention(got, ref, f"C3 block {b}")
            say(f"C3 block {b}: max-abs {np.abs(got - ref).max():.3e}, "
                f"rel-L2 {rel_l2(got, ref):.3e}")
            ids = sorted(int(x) for x in gs.ring.slot_ids() if x)
            assert ids == list(range(max(1, b - shape.W + 1), b + 1))


def _stage(L, shape, n_layers, staged=False):
    t = torch()
    s = shape
    stack = L.KVRingStack(n_layers, s.W, s.block_tokens, s.sink_tokens, s.heads, s.head_dim,
                          t.bfloat16 if s.dtype == "bf16" else t.float32, NOISE_LEVEL,
                          staged=staged)
    for l in range(n_layers):
        sk, sv = s.initial_sink(l)
        stack.sink_k_raw[l].copy_(to_dev(sk))
        stack.sink_v[l].copy_(to_dev(sv))
    table = t.empty(L.la_rope_table_bytes(s.Hl, s.Wl, s.head_dim) // 4, dtype=t.float32,
                    device="cuda")
    L.la_rope_table_fill(table, s.Hl, s.Wl, s.head_dim, THETA)
    return stack, table


def test_denoise_step_matches_oracle_and_per_op_path(L):
    """la_denoise_step over 3 layers and 6 blocks: each layer's attention equals the
    per-op C-ABI path bit for bit and the oracle within tolerance; the latent takes
    one Euler step per block."""
    t = torch()
    shape = si.MID_BF16
    s = shape
    n_layers = 3
    stack, table = _stage(L, shape, n_layers)
    blk = (s.block_tokens, s.heads, s.head_dim)
    outs = [t.empty(blk, dtype=t.bfloat16, device="cuda") for _ in range(n_layers)]
    qws, kws = t.empty(blk, dtype=t.bfloat16, device="cuda"), t.empty(blk, dtype=t.bfloat16, device="cuda")
    sws = t.empty((s.sink_tokens, s.heads, s.head_dim), dtype=t.bfloat16, device="cuda")
    per_op = [GpuLayerStream(shape, layer=l) for l in range(n_layers)]
    aws = L.AttnWorkspace(s.block_tokens, s.heads)  # one workspace for every layer
    oracles = [StreamOracle(shape, layer=l) for l in range(n_layers)]
    lat = si.latent(102, 0, si.TID_X, si.C4_LATENT_SHAPE)
    x = to_dev(lat)
    x_ref = lat.values.copy()
    for b in range(1, 7):
        ins = [s.block_inputs(l, b) for l in range(n_layers)]
        dev = [tuple(to_dev(z) for z in trip) for trip in ins]
        vel = si.latent(102, b, si.TID_VEL, si.C4_LATENT_SHAPE)
        veld = to_dev(vel)
        nsink = s.sink_tokens
        L.la_denoise_step(
            stack.states, b, [d[0] for d in dev], [d[1] for d in dev], [d[2] for d in dev], outs,
            qws, kws, sws, table, s.Hl, s.Wl, FRAMES_PER_BLOCK, SINK_DELTA, THETA,
            scale=softmax_scale(s.head_dim), attn_ws=aws,
            sink_k_new=[d[1][:nsink] for d in dev] if b == 1 else None,
            sink_v_new=[d[2][:nsink] for d in dev] if b == 1 else None,
            x=x, vel=veld, dt=-0.25)
        x_ref = euler_step(x_ref, vel.values, -0.25).astype(np.float32).astype(np.float64)
        for l in range(n_layers):
            per_op[l].step(b)
        t.cuda.synchronize()
        for l in range(n_layers):
            assert t.equal(outs[l].view(t.int16), per_op[l].out.view(t.int16)), (b, l)
            if b in (1, 2, 6):
                check_attention(to_f64(outs[l]), oracles[l].block_output(b), f"layer {l} block {b}")
        np.testing.assert_array_equal(x.cpu().numpy(), x_ref.astype(np.float32))
    for l in range(n_layers):
        assert stack.states[l].last_block == 6 and stack.states[l].sink_replaced == 1


@pytest.mark.timeout(600)
@pytest.mark.parametrize("shape_name", ["C2", "C3", "C5"])
def test_step_rotates_q_in_the_attention_with_the_same_bits(L, shape_name):
    """For bf16 rings la_denoise_step leaves Q's Rolling RoPE to the attention kernel:
    RoPE writes the block tokens' cos/sin (times q_scale) into q_rot_ws and the attention
    rotates the raw Q with them as it loads it.  At full size every output element
    equals the per-op path's (la_rope3d_rolling of Q into a workspace and of K into the
    ring's next slot, V copied there, then la_block_attn_fwd) bit for bit, over W + 2
    blocks: the sink replacement, the ring filling and evicting, and each block's own
    frame positions.  C3's window (W = 8) makes the longest joined run of keys, nine
    slots."""
    t = torch()
    s = getattr(si, shape_name)
    stack, table = _stage(L, s, 1, staged=True)
    per_op = GpuLayerStream(s, staged=True)
    blk = (s.block_tokens, s.heads, s.head_dim)
    out = t.empty(blk, dtype=t.bfloat16, device="cuda")
    qws = t.empty(blk, dtype=t.bfloat16, device="cuda")
    kws = t.empty(blk, dtype=t.bfloat16, device="cuda")
    sws = t.empty((s.sink_tokens, s.heads, s.head_dim), dtype=t.bfloat16, device="cuda")
    aws = L.AttnWorkspace(s.block_tokens, s.heads)
    nsink = s.sink_tokens
    for b in range(1, s.W + 3):
        q, k, v = per_op.block_dev(b)
        say(f"{shape_name} block {b}")
        L.la_denoise_step(stack.states, b, [q], [k], [v], [out], qws, kws, sws, table, s.Hl,
                          s.Wl, FRAMES_PER_BLOCK, SINK_DELTA, THETA,
                          scale=softmax_scale(s.head_dim), attn_ws=aws,
                          sink_k_new=[k[:nsink]] if b == 1 else None,
                          sink_v_new=[v[:nsink]] if b == 1 else None)
        per_op.step(b)
        t.cuda.synchronize()
        assert t.equal(out.view(t.int16), per_op.out.view(t.int16)), (shape_name, b)


@pytest.mark.parametrize("heads,staged", [(1, False), (1, True), (2, False), (2, True)])
def test_step_q_rotation_edge_heads(L, heads, staged):
    """The smallest head counts: with one head the step rotates Q in the RoPE launch (Q's
    cos/sin table, 512 bytes a token, would not fit the 256-byte rows of q_rot_ws); with
    two the table fills q_rot_ws exactly.  Plain and staged rings, W + 2 blocks of a
    ragged shape (390 rows: a partial query tile and partial key tiles in every segment),
    each block's output equal to the per-op path on the same kind of ring bit for bit
    and to the oracle within tolerance at three blocks."""
    t = torch()
    s = si.LayerShape(120 + heads, "bf16", heads=heads, head_dim=128, Hl=10, Wl=13, W=2)
    stack, table = _stage(L, s, 1, staged=staged)
    per_op = GpuLayerStream(s, staged=staged)
    oracle = StreamOracle(s)
    blk = (s.block_tokens, s.heads, s.head_dim)
    out = t.empty(blk, dtype=t.bfloat16, device="cuda")
    qws = t.empty(blk, dtype=t.bfloat16, device="cuda")
    kws = t.empty(blk, dtype=t.bfloat16, device="cuda")
    sws = t.empty((s.sink_tokens, s.heads, s.head_dim), dtype=t.bfloat16, device="cuda")
    aws = L.AttnWorkspace(s.block_tokens, s.heads)
    nsink = s.sink_tokens
    last = s.W + 2
    for b in range(1, last + 1):
        q, k, v = per_op.block_dev(b)
        L.la_denoise_step(stack.states, b, [q], [k], [v], [out], qws, kws, sws, table, s.Hl,
                          s.Wl, FRAMES_PER_BLOCK, SINK_DELTA, THETA,
                          scale=softmax_scale(s.head_dim), attn_ws=aws,
                          sink_k_new=[k[:nsink]] if b == 1 else None,
                          sink_v_new=[v[:nsink]] if b == 1 else None)
        per_op.step(b)
        t.cuda.synchronize()
        assert t.equal(out.view(t.int16), per_op.out.view(t.int16)), (heads, staged, b)
        if b in (1, 2, last):
            check_attention(to_f64(out), oracle.block_output(b), f"heads {heads} block {b}")


@pytest.mark.parametrize("case", ["mid_3_layers", "c2_1_layer"])
def test_staged_rings_fuse_the_append_with_the_same_bits(L, case):
    """Staged rings (W + 1 slots): la_denoise_step's RoPE launch writes each layer's
    rotated K straight into the ring's next slot and copies V there before the
    attention, and the append only records the block.  Every window block's K and V
    bytes equal those of the plain rings (which rotate into a workspace and copy both
    after the attention) bit for bit, through the sink replacement and W + 2
    evictions.  The outputs agree with the plain rings' within the attention bars (the
    staged block and its neighbouring slots are one run of keys, so the sums are
    rounded in another order), and the oracle checks them at three blocks."""
    t = torch()
    s = si.MID_BF16 if case == "mid_3_layers" else si.C2
    n_layers = 3 if case == "mid_3_layers" else 1
    plain, table = _stage(L, s, n_layers)
    staged, _ = _stage(L, s, n_layers, staged=True)
    blk = (s.block_tokens, s.heads, s.head_dim)
    ws = [[t.empty(blk, dtype=t.bfloat16, device="cuda") for _ in range(n_layers)]
          for _ in range(2)]
    qws, kws = t.empty(blk, dtype=t.bfloat16, device="cuda"), t.empty(blk, dtype=t.bfloat16, device="cuda")
    sws = t.empty((s.sink_tokens, s.heads, s.head_dim), dtype=t.bfloat16, device="cuda")
    aws = L.AttnWorkspace(s.block_tokens, s.heads)
    oracles = [StreamOracle(s, layer=l) for l in range(n_layers)]
    nsink = s.sink_tokens
    last = s.W + 3
    for b in range(1, last + 1):
        dev = [tuple(to_dev(z) for z in s.block_inputs(l, b)) for l in range(n_layers)]
        for stack, outs in ((plain, ws[0]), (staged, ws[1])):
            L.la_denoise_step(
                stack.states, b, [d[0] for d in dev], [d[1] for d in dev], [d[2] for d in dev],
                outs, qws, kws, sws, table, s.Hl, s.Wl, FRAMES_PER_BLOCK, SINK_DELTA, THETA,
                scale=softmax_scale(s.head_dim), attn_ws=aws,
                sink_k_new=[d[1][:nsink] for d in dev] if b == 1 else None,
                sink_v_new=[d[2][:nsink] for d in dev] if b == 1 else None)
        t.cuda.synchronize()
        for l in range(n_layers):
            check_attention(to_f64(ws[1][l]), to_f64(ws[0][l]), f"staged vs plain {b} {l}")
            for bid in range(max(1, b - s.W + 1), b + 1):
                ps, ss = (bid - 1) % s.W, (bid - 1) % (s.W + 1)
                assert int(plain.states[l].slot_block[ps]) == bid
                assert int(staged.states[l].slot_block[ss]) == bid
                for a, c in ((plain.k_slots, staged.k_slots), (plain.v_slots, staged.v_slots)):
                    assert t.equal(a[l, ps].view(t.int16), c[l, ss].view(t.int16)), (b, l, bid)
            if b in (1, 2, last) and (case == "mid_3_layers" or b == last):
                if case == "mid_3_layers":
                    check_attention(to_f64(ws[1][l]), oracles[l].block_output(b),
                                    f"staged layer {l} block {b}")
                else:
                    rows = np.unique(np.concatenate([[0, s.block_tokens - 1],
                                                     np.random.default_rng(b).integers(
                                                         0, s.block_tokens, 48)]))
                    ref, _ = oracle_block_all_heads(s, b, rows=rows)
                    check_attention(to_f64(ws[1][l])[rows], ref, f"staged C2 block {b}")
    for l in range(n_layers):
        assert staged.states[l].last_block == last and staged.states[l].sink_replaced == 1


def test_denoise_step_refuses_before_any_launch(L):
    t = torch()
    shape = si.SMALL_BF16
    s = shape
    stack, table = _stage(L, shape, 2)
    blk = (s.block_tokens, s.heads, s.head_dim)
    z = [t.zeros(blk, dtype=t.bfloat16, device="cuda") for _ in range(2)]
    ws = t.empty(blk, dtype=t.bfloat16, device="cuda")
    sws = t.empty((s.sink_tokens, s.heads, s.head_dim), dtype=t.bfloat16, device="cuda")
    before = [bytes(stack.states[l]) for l in range(2)]
    with pytest.raises(L.LAError):  # block 2 before block 1
        L.la_denoise_step(stack.states, 2, z, z, z, [ws, ws], ws, ws, sws, table, s.Hl, s.Wl,
                          scale=0.1)
    with pytest.raises(ValueError):  # wrong frame geometry: the table is too small for it
        L.la_denoise_step(stack.states, 1, z, z, z, [ws, ws], ws, ws, sws, table, s.Hl + 1, s.Wl,
                          scale=0.1)
    with pytest.raises(L.LAError) as e:  # blocks of 2 frames do not match the rings
        L.la_denoise_step(stack.states, 1, z, z, z, [ws, ws], ws, ws, sws, table, s.Hl, s.Wl,
                          frames_per_block=2, scale=0.1)
    assert e.value.status == L._lib.LA_ERR_SHAPE
    stack.states[1].noise_level = 0.5  # layers disagree on the noise level
    with pytest.raises(L.LAError):
        L.la_denoise_step(stack.states, 1, z, z, z, [ws, ws], ws, ws, sws, table, s.Hl, s.Wl,
                          scale=0.1)
    stack.states[1].noise_level = NOISE_LEVEL
    small = L.AttnWorkspace(s.block_tokens, s.heads)
    small.nbytes -= 256
    with pytest.raises(L.LAError):  # attention workspace below la_attn_workspace_bytes
        L.la_denoise_step(stack.states, 1, z, z, z, [ws, ws], ws, ws, sws, table, s.Hl, s.Wl,
                          scale=0.1, attn_ws=small)
    assert [bytes(stack.states[l]) for l in range(2)] == before


def test_checkpoint_restore_continues_bit_identically(L):
    """A stage's resumable state is the ring/sink index struct plus the device buffers;
    restoring it after block 4 and continuing gives the same bits as never stopping."""
    t = torch()
    shape = si.MID_BF16
    a = GpuLayerStream(shape)
    for b in range(1, 5):
        a.step(b)
    t.cuda.synchronize()
    saved_struct = bytes(a.ring.state)
    saved = [x.clone() for x in (a.ring.k_slots, a.ring.v_slots, a.ring.sink_k_raw, a.ring.sink_v)]
    for b in range(5, 9):
        a.step(b)
    t.cuda.synchronize()
    ref_out = a.out.clone()
    ref_slots = a.ring.k_slots.clone()

    bstream = GpuLayerStream(shape)
    for dst, src in zip((bstream.ring.k_slots, bstream.ring.v_slots, bstream.ring.sink_k_raw,
                         bstream.ring.sink_v), saved):
        dst.copy_(src)
    ctypes.memmove(ctypes.addressof(bstream.ring.state), saved_struct, len(saved_struct))
    # the struct holds device pointers: point them at the new buffers
    bstream.ring.state.k_slots = bstream.ring.k_slots.data_ptr()
    bstream.ring.state.v_slots = bstream.ring.v_slots.data_ptr()
    bstream.ring.state.sink_k_raw = bstream.ring.sink_k_raw.data_ptr()
    bstream.ring.state.sink_v = bstream.ring.sink_v.data_ptr()
    for b in range(5, 9):
        bstream.step(b)
    t.cuda.synchronize()
    assert t.equal(bstream.out.view(t.int16), ref_out.view(t.int16))
    assert t.equal(bstream.ring.k_slots.view(t.int16), ref_slots.view(t.int16))


def test_denoise_chain_four_stages_matches_oracle(L):
    """la_denoise_chain: one block through four timestep-forcing stages (noise levels
    1.0, 0.75, 0.5, 0.25, each stage with its own per-layer rings and inputs), five
    blocks.  Every stage's attention matches the float64 oracle of that stage's stream,
    and the latent equals four sequential float32 Euler steps bit for bit."""
    t = torch()
    s = si.SMALL_BF16
    n_layers, n_stages = 2, 4
    levels = [1.0 - 0.25 * i for i in range(n_stages)]
    stacks = []
    for i in range(n_stages):
        st = L.KVRingStack(n_layers, s.W, s.block_tokens, s.sink_tokens, s.heads, s.head_dim,
                           t.bfloat16, levels[i])
        for l in range(n_layers):
            sk, sv = s.initial_sink(i * n_layers + l)
            st.sink_k_raw[l].copy_(to_dev(sk))
            st.sink_v[l].copy_(to_dev(sv))
        stacks.append(st)
    table = t.empty(L.la_rope_table_bytes(s.Hl, s.Wl, s.head_dim) // 4, dtype=t.float32,
                    device="cuda")
    L.la_rope_table_fill(table, s.Hl, s.Wl, s.head_dim, THETA)
    blk = (s.block_tokens, s.heads, s.head_dim)
    outs = [[t.empty(blk, dtype=t.bfloat16, device="cuda") for _ in range(n_layers)]
            for _ in range(n_stages)]
    qws, kws = t.empty(blk, dtype=t.bfloat16, device="cuda"), t.empty(blk, dtype=t.bfloat16, device="cuda")
    sws = t.empty((s.sink_tokens, s.heads, s.head_dim), dtype=t.bfloat16, device="cuda")
    aws = L.AttnWorkspace(s.block_tokens, s.heads)
    oracles = [[StreamOracle(s, layer=i * n_layers + l, noise_level=levels[i])
                for l in range(n_layers)] for i in range(n_stages)]
    lat = si.latent(s.cfg_id, 0, si.TID_X, (16, 3, 8, 8))
    x = to_dev(lat)
    x_ref = lat.values.copy()
    for b in range(1, 6):
        stages, vels = [], []
        for i in range(n_stages):
            dev = [tuple(to_dev(z) for z in s.block_inputs(i * n_layers + l, b))
                   for l in range(n_layers)]
            vel = si.latent(s.cfg_id, 100 * b + i, si.TID_VEL, (16, 3, 8, 8))
            vels.append(vel)
            g = dict(rings=stacks[i].states, q_raw=[d[0] for d in dev], k_raw=[d[1] for d in dev],
                     v_raw=[d[2] for d in dev], attn_out=outs[i], vel=to_dev(vel), dt=-0.25)
            if b == 1:
                g["sink_k_new"] = [d[1][:s.sink_tokens] for d in dev]
                g["sink_v_new"] = [d[2][:s.sink_tokens] for d in dev]
            stages.append(g)
        L.la_denoise_chain(stages, b, qws, kws, sws, table, s.Hl, s.Wl, x=x,
                           frames_per_block=FRAMES_PER_BLOCK, sink_delta=SINK_DELTA, theta=THETA,
                           scale=softmax_scale(s.head_dim), attn_ws=aws)
        t.cuda.synchronize()
        for i in range(n_stages):
            x_ref = euler_step(x_ref, vels[i].values, -0.25).astype(np.float32).astype(np.float64)
            for l in range(n_layers):
                check_attention(to_f64(outs[i][l]), oracles[i][l].block_output(b),
                                f"stage {i} layer {l} block {b}")
                r = stacks[i].states[l]
                assert r.last_block == b and r.sink_replaced == 1 and r.noise_level == levels[i]
        np.testing.assert_array_equal(x.cpu().numpy(), x_ref.astype(np.float32))
