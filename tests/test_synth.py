"""The seeded input generator: bf16 rounding and the recipes' ranges."""
import math

import numpy as np
import pytest

import synth


def test_bf16_round_nearest_even_matches_torch():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(200000).astype(np.float32) * 10.0,
                        np.array([0.0, -0.0, 1.0, 1.00390625, 1.0 + 2**-8 + 2**-9, 3.4e38,
                                  -3.4e38, 1e-40, np.inf, -np.inf], dtype=np.float32)])
    # ties: exactly halfway between two bf16 values
    halves = (np.arange(1, 2000, dtype=np.uint32) << 16 | 0x8000).view(np.float32)
    x = np.concatenate([x, halves, -halves])
    mine = synth.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(mine, ref)
    # widening is exact
    back = synth.bf16_bits_to_f32(mine)
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_nan_maps_to_nan():
    b = synth.f32_to_bf16_bits(np.array([np.nan], dtype=np.float32))
    assert np.isnan(synth.bf16_bits_to_f32(b)[0])


def test_recipes_ranges_and_determinism():
    x = synth.config_inputs(1, T=64, B=2, H=3)
    y = synth.config_inputs(1, T=64, B=2, H=3)
    for n in ("r", "w", "k", "v", "kappa", "a"):
        assert x[n].dtype == np.uint16 and x[n].shape == (2, 64, 3, 64)
        assert np.array_equal(x[n], y[n])
    w = x.as_f32("w")
    lo = math.exp(-1 / math.sqrt(math.e))
    assert w.min() >= np.float32(lo) - 2**-8 and w.max() <= 1.0
    a = x.as_f32("a")
    assert a.min() >= 0.0 and a.max() <= 1.0
    kap = x.as_f32("kappa").astype(np.float64)
    nrm = np.linalg.norm(kap, axis=-1)
    assert np.abs(nrm - 1).max() < 2e-2  # unit before bf16 rounding
    assert x["s0"].shape == (2, 3, 64, 64) and abs(x["s0"].std() - 0.1) < 0.01


def test_config_recipes():
    c0 = synth.config_inputs(0)
    assert c0["r"].dtype == np.float32 and c0["s0"] is None and c0["epi"] is None
    kap = c0["kappa"].astype(np.float64)
    assert np.abs(np.linalg.norm(kap, axis=-1) - 1).max() < 1e-6
    c2 = synth.config_inputs(2, T=32, B=2)
    assert c2["epi"] is not None and c2["epi"]["r_k"].shape == (40, 64)
    assert c2["epi"]["eps"] == 64e-5
    w2 = c2.as_f32("w")
    assert w2.min() < 0.6 and w2.max() > 0.99
    c4 = synth.config_inputs(4, T=256)
    w4 = c4.as_f32("w")
    assert w4.min() >= 0.99 - 2**-8 and w4.max() <= 1.0
    assert c4.as_f32("a").mean() > 0.8
