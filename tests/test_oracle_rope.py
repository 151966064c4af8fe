"""Pins of the float64 3D RoPE oracle (closed forms, invariants, library routines)."""

import math

import numpy as np
import pytest

from oracle import band_frequencies, band_split, rope3d, StreamOracle, block_f0, SINK_DELTA
from seeded_inputs import LayerShape


def rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def test_golden_band_split_and_frequencies(golden):
    g = golden("rope_frequencies.json")
    for d, bands in g["bands"].items():
        assert band_split(int(d)) == tuple(bands)
    for c in g["cases"]:
        f = band_frequencies(c["head_dim"])[c["band"]][c["k"]]
        assert abs(f - c["freq"]) < 1e-15


@pytest.mark.parametrize("band", [0, 1, 2])
def test_golden_unit_turn_on_each_axis(golden, band):
    """A unit vector on the pair with frequency 0.01 turns by exactly 1 rad at position 100,
    and only the axis that owns the band moves it."""
    g = golden("rope_frequencies.json")
    d = 64
    k = {0: 6, 1: 5, 2: 5}[band]
    start = sum(band_split(d)[:band])
    dim = start + 2 * k
    # one frame of 101 x 101 tokens; choose the token whose coordinate on `band` is 100
    Hl = Wl = 101
    x = np.zeros((Hl * Wl, 1, d))
    x[:, 0, dim] = 1.0
    f0 = 100 if band == 0 else 0
    h = 100 if band == 1 else 0
    w = 100 if band == 2 else 0
    out = rope3d(x, 1, Hl, Wl, f0)
    tok = h * Wl + w
    assert abs(out[tok, 0, dim] - g["unit_turn"]["cos1"]) < 1e-13
    assert abs(out[tok, 0, dim + 1] - g["unit_turn"]["sin1"]) < 1e-13
    # the same pair on the token at the origin of that axis does not move
    if band != 0:
        assert out[0, 0, dim] == 1.0 and out[0, 0, dim + 1] == 0.0


def test_pairs_match_complex_multiplication():
    """Library routine: (x + iy) * exp(i a) with numpy complex arithmetic."""
    Hl, Wl, n_frames, H, d = 3, 5, 3, 2, 64
    x = rand((n_frames * Hl * Wl, H, d), 1)
    out = rope3d(x, n_frames, Hl, Wl, f0=7)
    j, hh, ww = np.meshgrid(np.arange(n_frames), np.arange(Hl), np.arange(Wl), indexing="ij")
    pos = [7 + j.ravel(), hh.ravel(), ww.ravel()]
    start = 0
    for p, width in zip(pos, band_split(d)):
        z = x[..., start:start + width:2] + 1j * x[..., start + 1:start + width:2]
        freq = np.array([10000.0 ** (-(2.0 * kk) / width) for kk in range(width // 2)])
        zr = z * np.exp(1j * p[:, None, None] * freq[None, None, :])
        np.testing.assert_allclose(out[..., start:start + width:2], zr.real, atol=1e-12)
        np.testing.assert_allclose(out[..., start + 1:start + width:2], zr.imag, atol=1e-12)
        start += width


def test_norm_preserved_and_origin_identity():
    x = rand((2 * 3 * 4, 3, 128), 2)
    out = rope3d(x, 2, 3, 4, f0=1234)
    np.testing.assert_allclose(np.linalg.norm(out, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-13)
    o0 = rope3d(x[:1], 1, 1, 1, f0=0)
    np.testing.assert_array_equal(o0, x[:1])


def test_composition_of_shifts():
    """R(a) R(b) = R(a + b) on the frame axis."""
    x = rand((1, 1, 128), 3)
    twice = rope3d(rope3d(x, 1, 1, 1, f0=40), 1, 1, 1, f0=2)
    once = rope3d(x, 1, 1, 1, f0=42)
    np.testing.assert_allclose(twice, once, atol=1e-12)


def test_relative_position_property():
    """<R(m) q, R(n) k> depends only on m - n on every axis."""
    q, k = rand((1, 1, 128), 4), rand((1, 1, 128), 5)
    def dot(fm, fn):
        return float(np.sum(rope3d(q, 1, 1, 1, fm) * rope3d(k, 1, 1, 1, fn)))
    assert abs(dot(10, 3) - dot(1010, 1003)) < 1e-10
    assert abs(dot(10, 3) - dot(3, 10)) > 1e-6  # sign of the offset matters


def test_rolling_sink_logits_shift_invariant():
    """Rolling RoPE: with the sink at f0(b)+delta, the sink logits of block b equal those of
    block b + D for the same raw Q and sink K (any D); a sink at a fixed position does not."""
    shape = LayerShape(900, "f32", heads=2, head_dim=64, Hl=3, Wl=4, W=2)
    orc = StreamOracle(shape)
    q = rand((shape.block_tokens, 2, 64), 6)
    sk = rand((shape.sink_tokens, 2, 64), 7)
    def logits(b, fixed_sink_pos=None):
        qr = orc.rot_block(q, b)
        if fixed_sink_pos is None:
            kr = orc.rot_sink(sk, b)
        else:
            kr = rope3d(sk, 1, shape.Hl, shape.Wl, fixed_sink_pos)
        return np.einsum("qhd,khd->hqk", qr, kr)
    base = logits(1)
    for D in (1, 199, 100000):
        np.testing.assert_allclose(logits(1 + D), base, atol=1e-9)
    assert np.max(np.abs(logits(50, fixed_sink_pos=SINK_DELTA) - base)) > 1e-2
    # the sink sits one frame before the block's first frame
    assert block_f0(1) + SINK_DELTA == -1 and block_f0(200) == 597


def test_rejects_bad_shapes():
    with pytest.raises(ValueError):
        rope3d(np.zeros((5, 1, 64)), 1, 2, 2, 0)
    with pytest.raises(ValueError):
        band_split(7)
