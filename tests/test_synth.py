"""The seeded input generator: determinism, shapes and bf16 rounding."""
import numpy as np
import pytest
import torch

from synth import CONFIGS, bf16_bits_from_f32, f32_from_bf16_bits, make_case, make_config


def test_bf16_rounding_matches_torch_round_to_nearest_even():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32),
                        np.array([1.00390625, 1.01171875, -1.00390625, 3.0e-39, 65504.0], np.float32)])
    ours = bf16_bits_from_f32(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = f32_from_bf16_bits(ours)
    assert np.array_equal(back, torch.from_numpy(ours.view(np.int16)).view(torch.bfloat16).float().numpy())


def test_generator_is_deterministic_and_blocked():
    a = make_case(5, D=16, V=40, G=2, lengths=[3000, 2500], dtype="bf16")
    b = make_case(5, D=16, V=40, G=2, lengths=[3000, 2500], dtype="bf16")
    for k in ("H", "W", "targets", "rewards", "noise_old", "noise_ref"):
        assert np.array_equal(getattr(a, k), getattr(b, k)), k
    assert a.H.shape == (5500, 16) and a.H.dtype == np.uint16
    assert a.cu.tolist() == [0, 3000, 5500]
    assert a.targets.min() >= 0 and a.targets.max() < 40


@pytest.mark.parametrize("cfg", [0, 1, 2, 3, 4])
def test_config_shapes_without_hidden_states(cfg):
    c = make_config(cfg, with_H=False) if cfg else make_config(0)
    spec = CONFIGS[cfg]
    assert c.W.shape == (spec["V"], spec["D"])
    assert c.S % c.G == 0
    expected_T = {0: 128, 2: 20480, 3: 110000, 4: 380000}
    if cfg in expected_T:
        assert c.T == expected_T[cfg]
    if cfg == 1:
        assert c.S == 64 and c.lengths.min() >= 256 and c.lengths.max() <= 1024
    if cfg == 4:
        assert c.S == 4 and c.lengths.min() >= 1
    assert np.all(c.mask == 1)
    w = f32_from_bf16_bits(c.W) if c.dtype == "bf16" else c.W
    assert abs(float(w.std()) - 0.02) < 0.002
