"""The seeded input generator: determinism, slicing, rounding and recipe."""
import numpy as np
import torch

import lmoe_synth as S


def test_deterministic_and_sliceable():
    cfg = S.CONFIGS["b05_n4096"]
    full = S.host_tensor(cfg, "w_g", 0, 100_000)
    again = S.host_tensor(cfg, "w_g", 0, 100_000)
    np.testing.assert_array_equal(full, again)
    np.testing.assert_array_equal(S.host_tensor(cfg, "w_g", 12_345, 777), full[12_345:12_345 + 777])
    other = S.host_tensor(cfg, "w_u", 0, 100_000)
    assert (full != other).mean() > 0.99


def test_bf16_rounding_is_round_to_nearest_even():
    rng = np.random.default_rng(0)
    a = rng.normal(size=100_000).astype(np.float32)
    a[:4] = [1.0 + 2**-8, 1.0 + 3 * 2**-8, -1.0 - 2**-8, 3.0]  # exact ties
    ref = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(S.f32_to_bf16_bits(a), ref)


def test_distribution_recipe():
    cfg = S.CONFIGS["toy_n128"]
    x = S.to_f64(S.host_tensor(cfg, "x"), "f32")
    assert abs(x.mean()) < 0.02 and abs(x.std() - 1) < 0.02
    wo = S.to_f64(S.host_tensor(cfg, "w_o"), "f32")
    assert abs(wo.std() * np.sqrt(cfg.ff_routed) - 1) < 0.01
    skew = S.CONFIGS["b05skew_n4096"]
    wr = S.to_f64(S.host_tensor(skew, "w_router"), "bf16").reshape(16, 768)
    assert abs(wr[:4].std() / wr[4:].std() - 3) < 0.1
    b = S.host_tensor(skew, "bias")
    np.testing.assert_allclose(b, (0.5 * (np.arange(16) / 15) ** 2).astype(np.float32))
    bu = S.host_tensor(S.CONFIGS["k3full_n64"], "bias")
    assert bu.shape == (896,) and bu.min() >= -0.01 and bu.max() <= 0.01 and bu.std() > 0.005


def test_flop_model():
    c = S.CONFIGS["k3full_n8192"]
    assert abs(c.flops() / 1e9 - 13213) < 5
    assert abs(S.CONFIGS["b05_n4096"].flops() / 1e9 - 96.74) < 0.05
