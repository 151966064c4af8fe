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
