"""Pins of the oracle's ring, sink, stream and flow-matching models."""

import numpy as np
import pytest

from oracle import (Ring, RingStateError, Sink, StreamOracle, euler_step, linear_path_point,
                    uniform_grid)
from seeded_inputs import LayerShape, SMALL_F32


def test_golden_ring_window(golden):
    g = golden("ring_window.json")
    r = Ring(g["W"], 0.5)
    ev = [r.append(b, np.full(2, b), np.full(2, -b), 0.5) for b in g["appends"]]
    assert ev == g["evicted"]
    assert r.ids() == g["final_ids"]
    assert r.slots() == {int(s): b for s, b in g["final_slots"].items()}


@pytest.mark.parametrize("W", [1, 2, 3, 8])
def test_ring_is_last_w_blocks_brute_force(W):
    r = Ring(W, 0.25)
    for n in range(1, 30):
        r.append(n, np.array([n]), np.array([10 * n]), 0.25)
        expect = [b for b in range(1, n + 1) if b > n - W]
        assert r.ids() == expect
        assert all(r.entry(b)[0][0] == b and r.entry(b)[1][0] == 10 * b for b in expect)
        slots = r.slots()
        assert sorted(slots) == sorted({(b - 1) % W for b in expect})
        assert all(r.noise_levels()[i] == 0.25 for i in range(len(r)))


def test_ring_refuses_out_of_order_and_wrong_noise_level():
    r = Ring(2, 0.5)
    r.append(1, np.zeros(1), np.zeros(1), 0.5)
    with pytest.raises(RingStateError):
        r.append(3, np.zeros(1), np.zeros(1), 0.5)
    with pytest.raises(RingStateError):
        r.append(2, np.zeros(1), np.zeros(1), 0.75)
    assert r.ids() == [1]


def test_sink_replaced_exactly_once():
    s = Sink(np.zeros((2, 3)), np.ones((2, 3)))
    s.replace(np.full((2, 3), 5.0), np.full((2, 3), 6.0))
    assert s.replaced and (s.k_raw == 5).all() and (s.v == 6).all()
    with pytest.raises(RingStateError):
        s.replace(np.zeros((2, 3)), np.zeros((2, 3)))
    assert (s.k_raw == 5).all() and (s.v == 6).all()


@pytest.mark.parametrize("shape", [SMALL_F32, LayerShape(901, "bf16", heads=2, head_dim=64, Hl=2, Wl=3, W=1)])
def test_stream_state_machine_equals_window_definition(shape):
    """The step-by-step run (Ring + Sink) and the direct window definition agree."""
    orc = StreamOracle(shape)
    n = shape.W + 4
    outs, ring, sink = orc.run(n, record=range(1, n + 1))
    for b in range(1, n + 1):
        np.testing.assert_allclose(outs[b], orc.block_output(b), atol=1e-12)
    assert ring.ids() == orc.window_ids(n + 1)
    assert sink.replaced


def test_aas_changes_block2_only_through_the_sink():
    """Block 1 sees the initial sink and block 2 the replacement; without the replacement
    block 2's output differs (negative control)."""
    shape = SMALL_F32
    orc = StreamOracle(shape)
    with_aas = orc.block_output(2)
    sink_init = orc.initial_sink()
    orc.sink_for = lambda b: sink_init  # plant: never replace
    without = orc.block_output(2)
    assert np.max(np.abs(with_aas - without)) > 1e-3


def test_key_count_matches_window_formula():
    shape = SMALL_F32
    orc = StreamOracle(shape)
    for b in (1, 2, shape.W + 1, shape.W + 5):
        n = shape.sink_tokens + len(orc.window_ids(b)) * shape.block_tokens + shape.block_tokens
        assert n == shape.nk(b)


def test_golden_euler_on_linear_path(golden):
    g = golden("euler_linear_path.json")
    x0, x1 = np.array(g["x0"]), np.array(g["x1"])
    xt = linear_path_point(x0, x1, g["t"])
    np.testing.assert_array_equal(xt, g["x_t"])
    np.testing.assert_array_equal(x1 - x0, g["v"])
    np.testing.assert_array_equal(euler_step(xt, x1 - x0, g["dt"]), g["x_next"])


def test_euler_walks_the_linear_path_exactly():
    """With dyadic x0, x1 every Euler step with v = x1 - x0 lands exactly on x_{t+dt}."""
    rng = np.random.default_rng(5)
    x0 = rng.integers(-8192, 8192, size=4096) / 1024.0
    x1 = rng.integers(-8192, 8192, size=4096) / 1024.0
    grid = uniform_grid(4)
    assert grid == [1.0, 0.75, 0.5, 0.25, 0.0]
    x = linear_path_point(x0, x1, grid[0])
    np.testing.assert_array_equal(x, x1)
    for t_prev, t_next in zip(grid[:-1], grid[1:]):
        x = euler_step(x, x1 - x0, t_next - t_prev)
        np.testing.assert_array_equal(x, linear_path_point(x0, x1, t_next))
        np.testing.assert_array_equal(x.astype(np.float32), linear_path_point(x0, x1, t_next).astype(np.float32))
    np.testing.assert_array_equal(x, x0)


def test_euler_fp32_rounding_is_single():
    """dt = -0.25 makes dt*v exact, so float64 x + dt*v rounded to float32 equals
    float32 arithmetic (one rounding): the fp32 kernel can match it bit for bit."""
    rng = np.random.default_rng(6)
    x = rng.standard_normal(100000).astype(np.float32)
    v = rng.standard_normal(100000).astype(np.float32)
    ref = euler_step(x, v, -0.25).astype(np.float32)
    np.testing.assert_array_equal(ref, x + np.float32(-0.25) * v)


# ---- ablation variants (NOTES Table 4: no Rolling RoPE, no AAS; clean / fixed-noise caches)
def _assemble(shape, own, owner, b, sink_pos, sink_kv):
    """Block b's attention assembled directly from the oracle's pinned pieces: own Q/K/V,
    the cache owner's window blocks, and the given raw sink rotated at sink_pos."""
    from oracle import attention_lse, rope3d
    f0 = lambda blk: 3 * (blk - 1)
    q, k, v = own.raw_block(b)
    keys = [rope3d(sink_kv[0], 1, shape.Hl, shape.Wl, sink_pos, own.theta)]
    vals = [sink_kv[1]]
    for b2 in range(max(1, b - shape.W), b):
        _, k2, v2 = owner.raw_block(b2)
        keys.append(rope3d(k2, 3, shape.Hl, shape.Wl, f0(b2), own.theta))
        vals.append(v2)
    keys.append(rope3d(k, 3, shape.Hl, shape.Wl, f0(b), own.theta))
    vals.append(v)
    qr = rope3d(q, 3, shape.Hl, shape.Wl, f0(b), own.theta)
    return attention_lse(qr, np.concatenate(keys), np.concatenate(vals), own.scale)[0]


@pytest.mark.parametrize("rolling,aas", [(False, True), (True, False), (False, False)])
def test_variant_state_machine_equals_window_definition(rolling, aas):
    shape = SMALL_F32
    orc = StreamOracle(shape, rolling=rolling, aas=aas)
    n = shape.W + 3
    outs, _, sink = orc.run(n, record=range(1, n + 1))
    for b in range(1, n + 1):
        np.testing.assert_allclose(outs[b], orc.block_output(b), atol=1e-12)
    assert sink.replaced == aas


def test_variant_outputs_from_their_definition():
    shape = SMALL_F32
    base = StreamOracle(shape)
    init = base.initial_sink()
    repl = base.replacement_sink()
    for b in (1, 2, shape.W + 2):
        # no Rolling RoPE: the sink stays at frame 0
        got = StreamOracle(shape, rolling=False).block_output(b)
        want = _assemble(shape, base, base, b, 0, init if b == 1 else repl)
        np.testing.assert_allclose(got, want, atol=1e-12)
        # no AAS: the initial sink at every block, rolling position
        got = StreamOracle(shape, aas=False).block_output(b)
        want = _assemble(shape, base, base, b, 3 * (b - 1) - 1, init)
        np.testing.assert_allclose(got, want, atol=1e-12)


def test_no_rolling_changes_outputs_after_block_1_negative_control():
    shape = SMALL_F32
    a, b_ = StreamOracle(shape), StreamOracle(shape, rolling=False)
    for blk in (2, 5):
        assert np.max(np.abs(a.block_output(blk) - b_.block_output(blk))) > 1e-4


def test_shared_cache_stream_reads_the_owner_cache_and_sink():
    """An attend-only stream (cache_layer = the writer's stream) sees the writer's window
    blocks and sink, and its own Q/K/V for the block itself."""
    shape = SMALL_F32
    writer = StreamOracle(shape, layer=7)
    reader = StreamOracle(shape, layer=3, cache_layer=7)
    for b in (1, 2, shape.W + 2):
        sink = writer.initial_sink() if b == 1 else writer.replacement_sink()
        want = _assemble(shape, StreamOracle(shape, layer=3), writer, b, 3 * (b - 1) - 1, sink)
        np.testing.assert_allclose(reader.block_output(b), want, atol=1e-12)
    with pytest.raises(ValueError):
        reader.run(2)
    # its own stream (cache_layer == layer) is the default stream
    np.testing.assert_allclose(StreamOracle(shape, layer=3, cache_layer=3).block_output(3),
                               StreamOracle(shape, layer=3).block_output(3), atol=0)
