"""Pins of the float64 attention oracle against things other than itself."""

import math

import numpy as np
import pytest
import torch

from oracle import attention, attention_lse


def rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


@pytest.mark.parametrize("nq,nk,h,d", [(5, 7, 2, 8), (17, 33, 3, 16), (1, 1, 1, 4), (48, 160, 2, 64)])
def test_matches_torch_sdpa_fp64(nq, nk, h, d):
    """Library routine: torch's scaled_dot_product_attention in float64 on the CPU."""
    q, k, v = rand((nq, h, d), 1), rand((nk, h, d), 2), rand((nk, h, d), 3)
    ours = attention(q, k, v, 1.0 / math.sqrt(d), row_chunk=4)
    tq, tk, tv = (torch.from_numpy(x).permute(1, 0, 2).unsqueeze(0) for x in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv)[0].permute(1, 0, 2).numpy()
    np.testing.assert_allclose(ours, ref, rtol=0, atol=1e-12)


def test_brute_force_python_loops():
    """Tiny case with math.exp in plain loops."""
    nq, nk, d = 3, 5, 4
    q, k, v = rand((nq, 1, d), 4), rand((nk, 1, d), 5), rand((nk, 1, d), 6)
    s = 0.37
    ours, lse = attention_lse(q, k, v, s)
    for i in range(nq):
        w = [math.exp(s * sum(q[i, 0, c] * k[j, 0, c] for c in range(d))) for j in range(nk)]
        z = sum(w)
        assert abs(math.log(z) - lse[0, i]) < 1e-12
        for c in range(d):
            assert abs(sum(w[j] * v[j, 0, c] for j in range(nk)) / z - ours[i, 0, c]) < 1e-12


def test_golden_two_keys(golden):
    g = golden("attention_two_keys.json")
    q = np.array(g["q"])[:, None, :]
    k = np.array(g["k"])[:, None, :]
    v = np.array(g["v"])[:, None, :]
    out, lse = attention_lse(q, k, v, g["scale"])
    np.testing.assert_allclose(out[:, 0, :], g["out"], atol=1e-14)
    np.testing.assert_allclose(lse[0], g["lse"], atol=1e-14)
    out2 = attention(q, k[::-1], v[::-1], g["scale"])
    np.testing.assert_allclose(out2[:, 0, :], g["out"], atol=1e-14)


def test_single_key_returns_v():
    q, k, v = rand((9, 2, 8), 7), rand((1, 2, 8), 8), rand((1, 2, 8), 9)
    out = attention(q, k, v, 0.5)
    np.testing.assert_allclose(out, np.broadcast_to(v, out.shape), atol=1e-14)


def test_identical_keys_give_mean_v():
    q = rand((4, 2, 8), 10)
    k = np.broadcast_to(rand((1, 2, 8), 11), (6, 2, 8)).copy()
    v = rand((6, 2, 8), 12)
    out = attention(q, k, v, 0.9)
    np.testing.assert_allclose(out, np.broadcast_to(v.mean(axis=0), out.shape), atol=1e-13)


def test_zero_query_gives_uniform_mean():
    k, v = rand((11, 3, 8), 13), rand((11, 3, 8), 14)
    out = attention(np.zeros((2, 3, 8)), k, v, 1.0)
    np.testing.assert_allclose(out, np.broadcast_to(v.mean(axis=0), out.shape), atol=1e-13)


def test_key_permutation_invariance():
    q, k, v = rand((7, 2, 16), 15), rand((29, 2, 16), 16), rand((29, 2, 16), 17)
    perm = np.random.default_rng(18).permutation(29)
    np.testing.assert_allclose(attention(q, k, v, 0.25), attention(q, k[perm], v[perm], 0.25),
                               atol=1e-13)


def test_heads_are_independent():
    q, k, v = rand((7, 3, 16), 19), rand((13, 3, 16), 20), rand((13, 3, 16), 21)
    full = attention(q, k, v, 0.25)
    one = attention(q[:, 1:2], k[:, 1:2], v[:, 1:2], 0.25)
    np.testing.assert_allclose(full[:, 1:2], one, atol=1e-14)


def test_segment_merge_identity():
    """Merging per-segment (max, sum, unnormalised output) equals one softmax.

    This is the identity a tiled/online-softmax kernel relies on, checked here
    against the oracle's monolithic result.
    """
    q = rand((6, 1, 8), 22)
    segs = [rand((n, 1, 8), 23 + i) for i, n in enumerate((4, 9, 1, 12))]
    vals = [rand((n, 1, 8), 40 + i) for i, n in enumerate((4, 9, 1, 12))]
    s = 0.6
    m = np.full(6, -np.inf)
    l = np.zeros(6)
    o = np.zeros((6, 8))
    for kk, vv in zip(segs, vals):
        sc = s * q[:, 0, :] @ kk[:, 0, :].T
        mn = np.maximum(m, sc.max(axis=1))
        a = np.exp(m - mn)
        p = np.exp(sc - mn[:, None])
        l = l * a + p.sum(axis=1)
        o = o * a[:, None] + p @ vv[:, 0, :]
        m = mn
    merged = o / l[:, None]
    mono, lse = attention_lse(q, np.concatenate(segs), np.concatenate(vals), s)
    np.testing.assert_allclose(merged, mono[:, 0, :], atol=1e-13)
    np.testing.assert_allclose(m + np.log(l), lse[0], atol=1e-13)


def test_rows_of_softmax_sum_to_one():
    """V = all ones makes every output exactly 1 (weights sum to 1)."""
    q, k = rand((5, 2, 8), 30), rand((17, 2, 8), 31)
    out = attention(q, k, np.ones((17, 2, 8)), 2.0)
    np.testing.assert_allclose(out, 1.0, atol=1e-13)


def test_chunking_does_not_change_result():
    q, k, v = rand((37, 2, 8), 32), rand((19, 2, 8), 33), rand((19, 2, 8), 34)
    np.testing.assert_array_equal(attention(q, k, v, 0.3, row_chunk=5),
                                  attention(q, k, v, 0.3, row_chunk=1000)[:37])


def test_rejects_empty_keys():
    with pytest.raises(ValueError):
        attention(np.zeros((2, 1, 4)), np.zeros((0, 1, 4)), np.zeros((0, 1, 4)), 1.0)
