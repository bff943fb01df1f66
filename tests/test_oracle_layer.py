"""Pins of the oracle's whole layer: dense/sparse equivalence, special cases
and a large-beta reduction to a composition of torch library routines."""
import numpy as np
import torch

import oracle as O

F = torch.nn.functional


def _tiny(rng, d=12, ell=6, R=5, k=2, ns=2, fr=7, fs=9, beta=4.0, beta2=25.0, eps=1e-6):
    a = {
        "w_down": rng.normal(size=(ell, d)) / np.sqrt(d),
        "w_router": rng.normal(size=(R, d)) / np.sqrt(d),
        "bias": rng.uniform(-0.05, 0.05, size=R),
        "w_g": rng.normal(size=(R, fr, ell)) / np.sqrt(ell),
        "w_u": rng.normal(size=(R, fr, ell)) / np.sqrt(ell),
        "w_o": rng.normal(size=(R, ell, fr)) / np.sqrt(fr),
        "sh_g": rng.normal(size=(ns, fs, d)) / np.sqrt(d),
        "sh_u": rng.normal(size=(ns, fs, d)) / np.sqrt(d),
        "sh_o": rng.normal(size=(ns, d, fs)) / np.sqrt(fs),
        "w_up": rng.normal(size=(d, ell)) / np.sqrt(ell),
        "rms_w": rng.uniform(0.5, 1.5, size=ell),
    }
    return a, O.weights_from_arrays(a, k, beta, beta2, eps)


def test_sparse_equals_dense_then_mask():
    rng = np.random.default_rng(0)
    for kw in [dict(), dict(R=8, k=3), dict(R=4, k=4), dict(ns=0)]:
        a, W = _tiny(rng, **kw)
        x = rng.normal(size=(23, 12))
        ys = O.forward(x, W)["y"]
        yd = O.forward(x, W, dense=True)["y"]
        np.testing.assert_allclose(ys, yd, rtol=1e-12, atol=1e-12)


def test_large_beta_layer_equals_torch_composition():
    rng = np.random.default_rng(1)
    k, eps = 2, 1e-6
    a, W = _tiny(rng, k=k, beta=1e8, beta2=1e8, eps=eps)
    x = rng.normal(size=(17, 12))
    got = O.forward(x, W)["y"]
    t = {n: torch.from_numpy(np.asarray(v)) for n, v in a.items()}
    X = torch.from_numpy(x)
    z = F.linear(X, t["w_down"])
    s = torch.sigmoid(F.linear(X, t["w_router"]))
    ids = torch.topk(s + t["bias"], k, dim=-1).indices
    sel = s.gather(-1, ids)
    p = sel / sel.sum(-1, keepdim=True)
    u = torch.zeros(17, 6, dtype=torch.float64)
    for n in range(17):
        for j in range(k):
            e = int(ids[n, j])
            h = F.silu(F.linear(z[n], t["w_g"][e])) * F.linear(z[n], t["w_u"][e])
            u[n] += p[n, j] * F.linear(h, t["w_o"][e])
    sh = sum(F.linear(F.silu(F.linear(X, t["sh_g"][j])) * F.linear(X, t["sh_u"][j]), t["sh_o"][j])
             for j in range(2))
    y = sh + F.linear(F.rms_norm(u, (6,), weight=t["rms_w"], eps=eps), t["w_up"])
    np.testing.assert_allclose(got, y.numpy(), rtol=1e-9, atol=1e-10)


def test_token_permutation_and_batch_split():
    rng = np.random.default_rng(2)
    _, W = _tiny(rng)
    x = rng.normal(size=(31, 12))
    y = O.forward(x, W)["y"]
    perm = rng.permutation(31)
    np.testing.assert_allclose(O.forward(x[perm], W)["y"], y[perm], rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(O.forward(x[:5], W)["y"], y[:5], rtol=1e-13, atol=1e-13)


def test_zero_gate_gives_shared_only_and_rmsnorm_of_zero():
    rng = np.random.default_rng(3)
    a, _ = _tiny(rng)
    a["w_g"] = np.zeros_like(a["w_g"])
    W = O.weights_from_arrays(a, 2)
    x = rng.normal(size=(9, 12))
    r = O.forward(x, W)
    assert np.all(r["u"] == 0)
    np.testing.assert_array_equal(r["y"], r["s_sh"])


def test_identical_experts_independent_of_routing():
    rng = np.random.default_rng(4)
    a, _ = _tiny(rng, R=6, k=3)
    for n in ("w_g", "w_u", "w_o"):
        a[n] = np.repeat(a[n][:1], 6, axis=0)
    W = O.weights_from_arrays(a, 3)
    x = rng.normal(size=(11, 12))
    r = O.forward(x, W)
    np.testing.assert_allclose(r["u"], O.situ(r["z"], a["w_g"][0], a["w_u"][0], a["w_o"][0], 4.0, 25.0),
                               rtol=1e-12, atol=1e-14)


def test_k_equals_R_mixture():
    rng = np.random.default_rng(5)
    a, W = _tiny(rng, R=4, k=4)
    x = rng.normal(size=(7, 12))
    r = O.forward(x, W)
    s = r["routes"].s
    mix = sum((s[:, e:e + 1] / s.sum(1, keepdims=True)) * O.situ(r["z"], a["w_g"][e], a["w_u"][e], a["w_o"][e], 4.0, 25.0)
              for e in range(4))
    np.testing.assert_allclose(r["u"], mix, rtol=1e-12, atol=1e-14)


def test_linearity_in_shared_down_projection():
    rng = np.random.default_rng(6)
    a, W = _tiny(rng)
    x = rng.normal(size=(8, 12))
    base = O.forward(x, W)
    a2 = dict(a, sh_o=2.5 * a["sh_o"])
    r2 = O.forward(x, O.weights_from_arrays(a2, 2))
    np.testing.assert_allclose(r2["s_sh"], 2.5 * base["s_sh"], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(r2["y"] - r2["s_sh"], base["y"] - base["s_sh"], rtol=1e-13, atol=1e-14)


def test_rmsnorm_properties():
    rng = np.random.default_rng(7)
    u = rng.normal(size=(10, 16)) * rng.uniform(0.01, 10, size=(10, 1))
    eps = 1e-6
    n = O.rmsnorm(u, np.ones(16), eps)
    ms = np.mean(u * u, axis=1)
    np.testing.assert_allclose(np.mean(n * n, axis=1), ms / (ms + eps), rtol=1e-13)
    np.testing.assert_allclose(n * np.sqrt(ms + eps)[:, None], u, rtol=1e-13)
    w = rng.uniform(0.5, 2, 16)
    ref = F.rms_norm(torch.from_numpy(u), (16,), weight=torch.from_numpy(w), eps=eps).numpy()
    np.testing.assert_allclose(O.rmsnorm(u, w, eps), ref, rtol=1e-13)


def test_external_routes_reproduce_own_routes():
    rng = np.random.default_rng(8)
    _, W = _tiny(rng)
    x = rng.normal(size=(12, 12))
    r = O.forward(x, W)
    r2 = O.forward(x, W, ids=r["ids"][:, ::-1].copy())  # order of a token's ids is irrelevant
    np.testing.assert_allclose(r2["y"], r["y"], rtol=1e-13, atol=1e-13)
