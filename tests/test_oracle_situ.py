"""Pins of the oracle's SiTU-GLU expert against the mathematics."""
import math

import numpy as np
import torch

import oracle as O

B1, B2 = 4.0, 25.0


def test_hidden_bounded_by_beta_product():
    vals = np.array([-1e4, -88.0, -3.0, -1e-30, 0.0, 1e-30, 3.0, 88.0, 1e4])
    ag, au = np.meshgrid(vals, vals)
    h = O.situ_hidden(ag, au, B1, B2)
    assert np.all(np.abs(h) < B1 * B2 + 1e-12)
    # saturation: gate -> beta1, up -> +-beta2
    assert O.situ_hidden(np.array([1e4]), np.array([1e4]), B1, B2)[0] == B1 * B2
    assert O.situ_hidden(np.array([1e4]), np.array([-1e4]), B1, B2)[0] == -B1 * B2
    # gate is odd-ish only through tanh; very negative gate pre-activation -> 0
    assert abs(O.situ_hidden(np.array([-1e4]), np.array([1.0]), B1, B2)[0]) < 1e-300


def _silu(a):
    return torch.nn.functional.silu(torch.from_numpy(a)).numpy()


def test_near_origin_series_bounds():
    # beta*tanh(a/beta) = a * t with 1 - a^2/(3 beta^2) <= t <= 1 - a^2/(3 beta^2) + 2 a^4/(15 beta^4)
    rng = np.random.default_rng(1)
    ag = rng.uniform(-0.1, 0.1, 500)
    au = rng.uniform(-0.1, 0.1, 500)
    ag = ag[np.abs(ag) > 1e-3]
    au = au[: ag.size]
    au = np.where(np.abs(au) < 1e-3, 1e-3, au)
    h = O.situ_hidden(ag, au, B1, B2)
    ratio = h / (_silu(ag) * au)  # = t1 * t2
    lo = (1 - ag**2 / (3 * B1**2)) * (1 - au**2 / (3 * B2**2))
    hi = (1 - ag**2 / (3 * B1**2) + 2 * ag**4 / (15 * B1**4)) * (1 - au**2 / (3 * B2**2) + 2 * au**4 / (15 * B2**4))
    assert np.all(ratio >= lo - 1e-15) and np.all(ratio <= hi + 1e-15)
    assert np.all(ratio < 1)  # the soft caps are really applied


def test_large_beta_limit_is_swiglu():
    rng = np.random.default_rng(4)
    v = rng.normal(size=(5, 6))
    wg, wu, wo = rng.normal(size=(9, 6)), rng.normal(size=(9, 6)), rng.normal(size=(6, 9))
    got = O.situ(v, wg, wu, wo, 1e8, 1e8)
    F = torch.nn.functional
    t = lambda a: torch.from_numpy(a)  # noqa: E731
    ref = F.linear(F.silu(F.linear(t(v), t(wg))) * F.linear(t(v), t(wu)), t(wo)).numpy()
    np.testing.assert_allclose(got, ref, rtol=1e-10, atol=1e-12)


def test_gate_uses_unscaled_sigmoid():
    # at a_g = beta1 * atanh(1/2): gate = beta1/2 * sigmoid(a_g)
    a = np.array([B1 * math.atanh(0.5)])
    gate = O.situ_hidden(a, np.array([1e9]), B1, B2)[0] / B2  # up saturates to beta2
    assert gate == np.float64(B1 / 2 / (1 + math.exp(-a[0]))) or abs(gate - B1 / 2 / (1 + math.exp(-a[0]))) < 1e-15
