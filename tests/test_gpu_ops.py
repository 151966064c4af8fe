"""GPU parity of the streaming kernels (RoPE, append/evict, sink replacement, Euler)
against the float64 oracle, through the C ABI."""

import numpy as np
import pytest

import seeded_inputs as si
from oracle import Ring, euler_step, linear_path_point, rope3d, uniform_grid

from gpu_helpers import (F32_MAX_ABS, NOISE_LEVEL, THETA, bf16_bits, check_rope_bf16, say,
                         to_dev, to_f64, torch)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def L():
    import streaming_causal_video_amd as lib
    lib.lib()
    return lib


# ------------------------------------------------------------------ Euler
@pytest.mark.parametrize("n", [0, 1, 3, 4, 1001, 16 * 3 * 60 * 104, (1 << 22) + 7])
def test_euler_bit_exact(L, n):
    t = torch()
    say(f"euler n={n}")
    x = si.latent(4, 1, si.TID_X, (n,))
    v = si.latent(4, 1, si.TID_VEL, (n,))
    xd, vd = to_dev(x), to_dev(v)
    L.la_fm_euler_step(xd, vd, -0.25)
    t.cuda.synchronize()
    got = xd.cpu().numpy()
    ref32 = x.storage + np.float32(-0.25) * v.storage
    np.testing.assert_array_equal(got, ref32)  # dt*v exact: one rounding on both sides
    ref64 = euler_step(x.values, v.values, -0.25)
    if n:
        assert np.max(np.abs(got - ref64)) <= F32_MAX_ABS
        np.testing.assert_array_equal(got, ref64.astype(np.float32))


def test_euler_unaligned_and_aliased(L):
    t = torch()
    n = 4099
    x = si.latent(4, 2, si.TID_X, (n + 1,))
    v = si.latent(4, 2, si.TID_VEL, (n + 1,))
    xd, vd = to_dev(x), to_dev(v)
    L.la_fm_euler_step(xd[1:], vd[1:], -0.25)  # 4-byte offset: scalar path
    t.cuda.synchronize()
    got = xd.cpu().numpy()
    np.testing.assert_array_equal(got[1:], x.storage[1:] + np.float32(-0.25) * v.storage[1:])
    assert got[0] == x.storage[0]
    xd2 = to_dev(x)
    L.la_fm_euler_step(xd2, xd2, 0.5)  # x == v
    t.cuda.synchronize()
    np.testing.assert_array_equal(xd2.cpu().numpy(), x.storage + np.float32(0.5) * x.storage)


def test_euler_walks_linear_path_on_gpu(L):
    """Four GPU Euler steps with v = x1 - x0 from x1 (t = 1) land exactly on x0 (t = 0)."""
    t = torch()
    rng = np.random.default_rng(3)
    n = 1 << 20
    x0 = (rng.integers(-8192, 8192, size=n) / 1024.0).astype(np.float32)
    x1 = (rng.integers(-8192, 8192, size=n) / 1024.0).astype(np.float32)
    xd = t.from_numpy(x1.copy()).cuda()
    vd = t.from_numpy(x1 - x0).cuda()
    grid = uniform_grid(4)
    for a, b in zip(grid[:-1], grid[1:]):
        L.la_fm_euler_step(xd, vd, b - a)
        t.cuda.synchronize()
        np.testing.assert_array_equal(xd.cpu().numpy(),
                                      linear_path_point(x0, x1, b).astype(np.float32))


# ------------------------------------------------------------------ RoPE
def _rope_case(L, shape, f0, delta=-1, heads=None, inplace=False):
    t = torch()
    s = shape
    q, k, _ = s.block_inputs(0, 1)
    sk, _ = s.initial_sink(0)
    table = t.empty(L.la_rope_table_bytes(s.Hl, s.Wl, s.head_dim) // 4, dtype=t.float32,
                    device="cuda")
    L.la_rope_table_fill(table, s.Hl, s.Wl, s.head_dim, THETA)
    qd, kd, skd = to_dev(q), to_dev(k), to_dev(sk)
    if inplace:
        qo, ko, sko = qd, kd, skd
    else:
        qo, ko, sko = t.empty_like(qd), t.empty_like(kd), t.empty_like(skd)
    L.la_rope3d_rolling(qd, qo, kd, ko, 3, f0, skd, sko, delta, table, s.Hl, s.Wl, s.heads,
                        s.head_dim, THETA)
    t.cuda.synchronize()
    hs = list(range(s.heads)) if heads is None else heads
    for name, raw, out, nf, pos in (("q", q, qo, 3, f0), ("k", k, ko, 3, f0),
                                    ("sink", sk, sko, 1, f0 + delta)):
        ref = rope3d(raw.values[:, hs, :], nf, s.Hl, s.Wl, pos, THETA)
        if s.dtype == "bf16":
            check_rope_bf16(bf16_bits(out)[:, hs, :], ref, raw.values[:, hs, :], name)
        else:
            err = np.abs(to_f64(out)[:, hs, :] - ref).max()
            assert err <= F32_MAX_ABS, f"{name}: max-abs {err:.3e}"


@pytest.mark.parametrize("f0", [0, 3, 597, 2997, 30000, 300000])
def test_rope_f32_c1(L, f0):
    say(f"rope C1 f0={f0}")
    _rope_case(L, si.C1, f0)


@pytest.mark.parametrize("shape", [si.SMALL_BF16, si.MID_BF16, si.SMALL_F32, si.SMALL_F32_D128])
@pytest.mark.parametrize("f0", [0, 597, 299997])
def test_rope_small(L, shape, f0):
    say(f"rope {shape.cfg_id} f0={f0}")
    _rope_case(L, shape, f0)


def test_rope_in_place(L):
    _rope_case(L, si.MID_BF16, 123, inplace=True)


@pytest.mark.parametrize("shape,f0", [(si.C2, 597), (si.C5, 2997)])
def test_rope_full_size_sampled_heads(L, shape, f0):
    say(f"rope full size cfg {shape.cfg_id}")
    _rope_case(L, shape, f0, heads=[0, 13, shape.heads - 1])


# ------------------------------------------------------------------ append / evict / sink
def _ring(L, shape):
    t = torch()
    dt = t.bfloat16 if shape.dtype == "bf16" else t.float32
    return L.KVRing(shape.W, shape.block_tokens, shape.sink_tokens, shape.heads, shape.head_dim,
                    dt, NOISE_LEVEL)


@pytest.mark.parametrize("shape", [si.SMALL_BF16, si.MID_BF16, si.SMALL_F32, si.C1])
def test_append_evict_last_w_blocks_bit_exact(L, shape):
    t = torch()
    say(f"append cfg {shape.cfg_id}")
    ring = _ring(L, shape)
    model = Ring(shape.W, NOISE_LEVEL)
    blocks = {}
    for b in range(1, 3 * shape.W + 3):
        _, k, v = shape.block_inputs(0, b)
        kd, vd = to_dev(k), to_dev(v)
        blocks[b] = (k.storage, v.storage)
        ev = L.la_kvcache_append_evict(ring.state, kd, vd, b, NOISE_LEVEL)
        ev_model = model.append(b, k.storage, v.storage, NOISE_LEVEL)
        assert ev == (ev_model or 0)
        t.cuda.synchronize()
        assert ring.count == len(model)
        slots = model.slots()
        assert {s: int(ring.state.slot_block[s]) for s in slots} == slots
        view = np.uint16 if shape.dtype == "bf16" else np.float32
        ks = ring.k_slots.view(t.int16 if view is np.uint16 else t.float32).cpu().numpy().view(view)
        vs = ring.v_slots.view(t.int16 if view is np.uint16 else t.float32).cpu().numpy().view(view)
        for s, bid in slots.items():
            np.testing.assert_array_equal(ks[s], blocks[bid][0])
            np.testing.assert_array_equal(vs[s], blocks[bid][1])
    with pytest.raises(L.LAError):
        L.la_kvcache_append_evict(ring.state, kd, vd, b + 2, NOISE_LEVEL)
    with pytest.raises(L.LAError):
        L.la_kvcache_append_evict(ring.state, kd, vd, b + 1, NOISE_LEVEL + 0.25)
    assert ring.state.last_block == b


@pytest.mark.parametrize("shape", [si.SMALL_BF16, si.SMALL_F32])
def test_staged_append_takes_halves_already_in_place(L, shape):
    """A staged ring (W + 1 slots) places block b in slot (b - 1) mod (W + 1); an append
    whose K and/or V is the destination slot itself (written there beforehand, as the
    fused step does with K) copies only the other half.  The window's bytes and ids
    match the oracle's deque bit for bit for every mix of in-place halves."""
    t = torch()
    dt = t.bfloat16 if shape.dtype == "bf16" else t.float32
    W = shape.W
    ring = L.KVRing(W, shape.block_tokens, shape.sink_tokens, shape.heads, shape.head_dim, dt,
                    NOISE_LEVEL, staged=True)
    model = Ring(W, NOISE_LEVEL)
    blocks = {}
    view = np.uint16 if shape.dtype == "bf16" else np.float32
    tv = t.int16 if view is np.uint16 else t.float32
    for b in range(1, 3 * W + 4):
        _, k, v = shape.block_inputs(0, b)
        kd, vd = to_dev(k), to_dev(v)
        blocks[b] = (k.storage, v.storage)
        slot = (b - 1) % (W + 1)
        kptr, vptr = L.la_kvring_next_slot(ring.state)
        assert kptr == ring.k_slots[slot].data_ptr() and vptr == ring.v_slots[slot].data_ptr()
        mode = b % 3  # 0: both in place, 1: K in place, 2: V in place
        ksrc, vsrc = kd, vd
        if mode in (0, 1):
            ring.k_slots[slot].copy_(kd)
            ksrc = ring.k_slots[slot]
        if mode in (0, 2):
            ring.v_slots[slot].copy_(vd)
            vsrc = ring.v_slots[slot]
        ev = L.la_kvcache_append_evict(ring.state, ksrc, vsrc, b, NOISE_LEVEL)
        assert ev == (model.append(b, k.storage, v.storage, NOISE_LEVEL) or 0)
        t.cuda.synchronize()
        ks = ring.k_slots.view(tv).cpu().numpy().view(view)
        vs = ring.v_slots.view(tv).cpu().numpy().view(view)
        assert ring.count == len(model)
        for bid in model.ids():
            s_ = (bid - 1) % (W + 1)
            assert int(ring.state.slot_block[s_]) == bid
            np.testing.assert_array_equal(ks[s_], blocks[bid][0])
            np.testing.assert_array_equal(vs[s_], blocks[bid][1])


def test_append_full_size_c5(L):
    t = torch()
    s = si.C5
    say("append C5 full size")
    ring = _ring(L, s)
    for b in range(1, s.W + 2):
        _, k, v = s.block_inputs(0, b)
        kd, vd = to_dev(k), to_dev(v)
        L.la_kvcache_append_evict(ring.state, kd, vd, b, NOISE_LEVEL)
        t.cuda.synchronize()
        slot = (b - 1) % s.W
        assert t.equal(ring.k_slots[slot], kd) and t.equal(ring.v_slots[slot], vd)
    assert [int(x) for x in ring.slot_ids()] == [5, 2, 3, 4]


def test_sink_replaced_exactly_once(L):
    t = torch()
    s = si.MID_BF16
    ring = _ring(L, s)
    sk, sv = s.initial_sink(0)
    ring.sink_k_raw.copy_(to_dev(sk))
    ring.sink_v.copy_(to_dev(sv))
    _, k, v = s.block_inputs(0, 1)
    kd, vd = to_dev(k), to_dev(v)
    with pytest.raises(L.LAError):  # before block 1 has been appended
        L.la_sink_replace(ring.state, kd[: s.sink_tokens], vd[: s.sink_tokens])
    L.la_kvcache_append_evict(ring.state, kd, vd, 1, NOISE_LEVEL)
    L.la_sink_replace(ring.state, kd[: s.sink_tokens], vd[: s.sink_tokens])
    t.cuda.synchronize()
    assert ring.state.sink_replaced == 1
    assert t.equal(ring.sink_k_raw, kd[: s.sink_tokens]) and t.equal(ring.sink_v, vd[: s.sink_tokens])
    _, k2, v2 = s.block_inputs(0, 2)
    with pytest.raises(L.LAError):
        L.la_sink_replace(ring.state, to_dev(k2)[: s.sink_tokens], to_dev(v2)[: s.sink_tokens])
    t.cuda.synchronize()
    assert t.equal(ring.sink_k_raw, kd[: s.sink_tokens]) and t.equal(ring.sink_v, vd[: s.sink_tokens])
