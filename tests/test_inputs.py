"""The seeded input generator: determinism and bf16 round-to-nearest-even."""

import numpy as np
import torch

import seeded_inputs as si


def test_golden_bf16_rne(golden):
    g = golden("bf16_rne.json")
    for c in g["cases"]:
        assert int(si.f64_to_bf16_bits(np.array([c["x"]]))[0]) == c["bits"], c


def test_bf16_matches_torch_conversion_of_float32():
    """Library routine: torch's float32 -> bfloat16 cast rounds to nearest even; on
    float32-representable inputs the single rounding from float64 must agree."""
    x = np.random.default_rng(0).standard_normal(200000).astype(np.float32)
    x = np.concatenate([x, x * 1e-20, x * 1e20])
    ours = si.f64_to_bf16_bits(x.astype(np.float64))
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    np.testing.assert_array_equal(si.bf16_bits_to_f64(ours),
                                  torch.from_numpy(x).to(torch.bfloat16).double().numpy())


def test_seeded_and_deterministic():
    a = si.tensor(2, 0, 1, si.TID_Q, (4, 2, 8), "bf16")
    b = si.tensor(2, 0, 1, si.TID_Q, (4, 2, 8), "bf16")
    c = si.tensor(2, 0, 1, si.TID_K, (4, 2, 8), "bf16")
    np.testing.assert_array_equal(a.storage, b.storage)
    assert not np.array_equal(a.storage, c.storage)
    f = si.tensor(1, 0, 1, si.TID_Q, (4, 2, 8), "f32")
    assert f.storage.dtype == np.float32
    np.testing.assert_array_equal(f.values, f.storage.astype(np.float64))


def test_config_sizes():
    assert si.C2.block_tokens == 4680 and si.C2.sink_tokens == 1560
    assert si.C2.nk(5) == 24960 and si.C2.nk(1) == 6240
    assert si.C3.nk(200) == 43680
    assert si.C5.nk(10) == 56320  # sink + W blocks + the block itself
    assert si.C1.nk(1) == 64 and si.C1.nk(2) == 112 and si.C1.nk(10) == 160
    assert si.C3.entry(1) == 0 and si.C3.entry(17) == 0 and si.C3.entry(200) == 199 % 16
