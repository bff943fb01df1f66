"""Pins of the oracle's routed-block backward (``routed_backward``) and the
SiTU-GLU derivative (``situ_hidden_grad``) against the mathematics: central
finite differences of the pinned forward, torch autograd of an independent
dense torch composition, and the exact zeros of experts without pairs."""
import numpy as np
import pytest
import torch

import oracle as O

B1, B2 = 4.0, 25.0


def _case(seed, N=5, ell=6, ff=4, R=4, k=2, scale=0.7, skip_expert=None):
    rng = np.random.default_rng(seed)
    z = rng.normal(0, 1, (N, ell))
    wg = rng.normal(0, scale, (R, ff, ell))
    wu = rng.normal(0, scale, (R, ff, ell))
    wo = rng.normal(0, scale, (R, ell, ff))
    experts_allowed = [e for e in range(R) if e != skip_expert]
    ids = np.stack([rng.choice(experts_allowed, size=k, replace=False) for _ in range(N)])
    p = rng.uniform(0.1, 1.0, (N, k))
    du = rng.normal(0, 1, (N, ell))
    return z, wg, wu, wo, ids, p, du


def _loss(z, wg, wu, wo, ids, p, du, R):
    u = O.routed_sparse(z, ids, p, lambda e: (wg[e], wu[e], wo[e]), R, B1, B2)
    return float(np.sum(du * u))


def _fd(f, x, idx, h=1e-6):
    xp, xm = x.copy(), x.copy()
    xp[idx] += h
    xm[idx] -= h
    return (f(xp) - f(xm)) / (2 * h)


def test_situ_grad_matches_central_differences():
    rng = np.random.default_rng(3)
    ag = np.concatenate([rng.uniform(-6, 6, 200), [-40.0, -12.0, 0.0, 12.0, 40.0]])
    au = np.concatenate([rng.uniform(-80, 80, 200), [-200.0, -30.0, 0.0, 30.0, 200.0]])
    dg, du = O.situ_hidden_grad(ag, au, B1, B2)
    h = 1e-6
    fd_g = (O.situ_hidden(ag + h, au, B1, B2) - O.situ_hidden(ag - h, au, B1, B2)) / (2 * h)
    fd_u = (O.situ_hidden(ag, au + h, B1, B2) - O.situ_hidden(ag, au - h, B1, B2)) / (2 * h)
    np.testing.assert_allclose(dg, fd_g, rtol=1e-6, atol=1e-7)
    np.testing.assert_allclose(du, fd_u, rtol=1e-6, atol=1e-7)


def test_situ_grad_equals_torch_autograd():
    rng = np.random.default_rng(4)
    ag = torch.tensor(rng.uniform(-8, 8, 300), dtype=torch.float64, requires_grad=True)
    au = torch.tensor(rng.uniform(-60, 60, 300), dtype=torch.float64, requires_grad=True)
    h = (B1 * torch.tanh(ag / B1) * torch.sigmoid(ag)) * (B2 * torch.tanh(au / B2))
    h.sum().backward()
    dg, du = O.situ_hidden_grad(ag.detach().numpy(), au.detach().numpy(), B1, B2)
    np.testing.assert_allclose(dg, ag.grad.numpy(), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(du, au.grad.numpy(), rtol=1e-12, atol=1e-14)


def test_situ_grad_large_beta_is_swiglu_grad():
    # beta -> inf: h -> silu(a_g) * a_u, so dh/da_g -> silu'(a_g) a_u and dh/da_u -> silu(a_g)
    rng = np.random.default_rng(5)
    ag = torch.tensor(rng.uniform(-5, 5, 100), dtype=torch.float64, requires_grad=True)
    au = torch.tensor(rng.uniform(-5, 5, 100), dtype=torch.float64)
    torch.nn.functional.silu(ag).sum().backward()
    dg, du = O.situ_hidden_grad(ag.detach().numpy(), au.numpy(), 1e7, 1e7)
    np.testing.assert_allclose(dg, ag.grad.numpy() * au.numpy(), rtol=1e-9, atol=1e-12)
    np.testing.assert_allclose(du, torch.nn.functional.silu(ag).detach().numpy(), rtol=1e-9, atol=1e-12)


@pytest.mark.parametrize("seed", [0, 1])
def test_routed_backward_matches_finite_differences(seed):
    R = 4
    z, wg, wu, wo, ids, p, du = _case(seed, R=R)
    g = O.routed_backward(z, ids, p, lambda e: (wg[e], wu[e], wo[e]), R, B1, B2, du)
    rng = np.random.default_rng(100 + seed)
    for _ in range(6):
        i = tuple(rng.integers(0, s) for s in z.shape)
        assert abs(_fd(lambda zz: _loss(zz, wg, wu, wo, ids, p, du, R), z, i) - g.dz[i]) < 1e-6
        i = tuple(rng.integers(0, s) for s in p.shape)
        assert abs(_fd(lambda pp: _loss(z, wg, wu, wo, ids, pp, du, R), p, i) - g.dp[i]) < 1e-6
        for which, arr in ((0, wg), (1, wu), (2, wo)):
            i = tuple(rng.integers(0, s) for s in arr.shape)

            def f(a, which=which):
                ws = [wg, wu, wo]
                ws[which] = a
                return _loss(z, *ws, ids, p, du, R)
            assert abs(_fd(f, arr, i) - g.dw[i[0]][which][i[1:]]) < 1e-6


def test_routed_backward_equals_torch_dense_autograd():
    """The dense-then-mask helper of the pages' tests, written with torch
    ops and differentiated by torch autograd (fp64, CPU)."""
    R, k = 6, 3
    z, wg, wu, wo, ids, p, du = _case(7, N=9, ell=8, ff=5, R=R, k=k)
    T = lambda a: torch.tensor(a, dtype=torch.float64, requires_grad=True)  # noqa: E731
    zt, pt, wgt, wut, wot = T(z), T(p), T(wg), T(wu), T(wo)
    outs = []
    for e in range(R):
        ag, au = zt @ wgt[e].T, zt @ wut[e].T
        h = (B1 * torch.tanh(ag / B1) * torch.sigmoid(ag)) * (B2 * torch.tanh(au / B2))
        outs.append(h @ wot[e].T)
    allo = torch.stack(outs, dim=1)  # [N, R, ell]
    u = torch.zeros_like(zt)
    rows = torch.arange(z.shape[0])
    for j in range(k):
        u = u + pt[:, j:j + 1] * allo[rows, torch.as_tensor(ids[:, j])]
    (u * torch.as_tensor(du)).sum().backward()
    g = O.routed_backward(z, ids, p, lambda e: (wg[e], wu[e], wo[e]), R, B1, B2, du)
    np.testing.assert_allclose(g.dz, zt.grad.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(g.dp, pt.grad.numpy(), rtol=1e-11, atol=1e-12)
    for e in range(R):
        np.testing.assert_allclose(g.dw[e][0], wgt.grad[e].numpy(), rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(g.dw[e][1], wut.grad[e].numpy(), rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(g.dw[e][2], wot.grad[e].numpy(), rtol=1e-11, atol=1e-12)


def test_unselected_expert_gets_exact_zero_grads():
    R = 5
    z, wg, wu, wo, ids, p, du = _case(11, N=7, R=R, k=2, skip_expert=3)
    assert not (ids == 3).any()
    g = O.routed_backward(z, ids, p, lambda e: (wg[e], wu[e], wo[e]), R, B1, B2, du)
    for a in g.dw[3]:
        assert np.all(a == 0.0)
    assert any(np.any(a != 0) for e in (0, 1, 2, 4) for a in g.dw[e])


def test_routed_backward_subset_and_empty():
    R = 4
    z, wg, wu, wo, ids, p, du = _case(12, R=R)
    full = O.routed_backward(z, ids, p, lambda e: (wg[e], wu[e], wo[e]), R, B1, B2, du)
    part = O.routed_backward(z, ids, p, lambda e: (wg[e], wu[e], wo[e]), R, B1, B2, du, want=[1, 2])
    assert sorted(part.dw) == [1, 2]
    for e in (1, 2):
        for a, b in zip(full.dw[e], part.dw[e]):
            assert np.array_equal(a, b)
    assert np.array_equal(full.dz, part.dz) and np.array_equal(full.dp, part.dp)
    empty = O.routed_backward(np.zeros((0, 6)), np.zeros((0, 2), dtype=np.int64), np.zeros((0, 2)),
                              lambda e: (wg[e], wu[e], wo[e]), R, B1, B2, np.zeros((0, 6)))
    assert empty.dz.shape == (0, 6) and all(np.all(a == 0) for v in empty.dw.values() for a in v)


def test_only_want_restricts_to_wanted_experts():
    R = 4
    z, wg, wu, wo, ids, p, du = _case(13, R=R)
    full = O.routed_backward(z, ids, p, lambda e: (wg[e], wu[e], wo[e]), R, B1, B2, du)
    e = int(ids[0, 0])
    only = O.routed_backward(z, ids, p, lambda x: (wg[x], wu[x], wo[x]), R, B1, B2, du, want=[e], only_want=True)
    for a, b in zip(full.dw[e], only.dw[e]):
        assert np.array_equal(a, b)
    # dp of the wanted expert's pairs is complete, the others are left at zero
    mask = ids == e
    assert np.array_equal(only.dp[mask], full.dp[mask]) and np.all(only.dp[~mask] == 0)


# ------------------------------------------------------------ whole layer


def _tiny_layer(seed, d=10, ell=6, R=5, k=2, ns=2, fr=4, fs=7):
    rng = np.random.default_rng(seed)
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
    x = rng.normal(size=(6, d))
    dy = rng.normal(size=(6, d))
    return a, x, dy, k


def test_rmsnorm_backward_equals_torch_autograd():
    rng = np.random.default_rng(21)
    u = torch.tensor(rng.normal(size=(5, 8)), dtype=torch.float64, requires_grad=True)
    w = torch.tensor(rng.uniform(0.5, 1.5, 8), dtype=torch.float64, requires_grad=True)
    dr = rng.normal(size=(5, 8))
    r = torch.nn.functional.rms_norm(u, (8,), w, eps=1e-6)
    (r * torch.as_tensor(dr)).sum().backward()
    du, dw = O.rmsnorm_backward(u.detach().numpy(), w.detach().numpy(), 1e-6, dr)
    np.testing.assert_allclose(du, u.grad.numpy(), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(dw, w.grad.numpy(), rtol=1e-12, atol=1e-13)


def test_layer_backward_matches_finite_differences():
    a, x, dy, k = _tiny_layer(22)
    W = O.weights_from_arrays(a, k)
    ids = O.forward(x, W)["ids"]
    g = O.layer_backward(x, W, dy, ids=ids)

    def loss(aa, xx):
        return float(np.sum(dy * O.forward(xx, O.weights_from_arrays(aa, k), ids=ids)["y"]))

    rng = np.random.default_rng(23)
    h = 1e-6
    for _ in range(4):
        i = tuple(rng.integers(0, s) for s in x.shape)
        xp, xm = x.copy(), x.copy()
        xp[i] += h
        xm[i] -= h
        assert abs((loss(a, xp) - loss(a, xm)) / (2 * h) - g["x"][i]) < 1e-6
        for name in ("w_down", "w_router", "w_up", "rms_w", "sh_g", "sh_u", "sh_o", "w_g", "w_u", "w_o"):
            arr = a[name]
            i = tuple(rng.integers(0, s) for s in arr.shape)
            ap, am = dict(a), dict(a)
            ap[name], am[name] = arr.copy(), arr.copy()
            ap[name][i] += h
            am[name][i] -= h
            fd = (loss(ap, x) - loss(am, x)) / (2 * h)
            if name in ("w_g", "w_u", "w_o"):
                got = g["routed"][i[0]][("w_g", "w_u", "w_o").index(name)][i[1:]]
            else:
                got = g[name][i]
            assert abs(fd - got) < 1e-6, (name, fd, got)


def test_layer_backward_equals_torch_autograd():
    """The layer written with torch library ops (F.linear, sigmoid, a gather
    over the fixed routes, SiTU, F.rms_norm) and differentiated by autograd."""
    a, x, dy, k = _tiny_layer(24, R=6, k=3)
    W = O.weights_from_arrays(a, k)
    ids = O.forward(x, W)["ids"]
    T = {n: torch.tensor(v, dtype=torch.float64, requires_grad=n != "bias") for n, v in a.items()}
    xt = torch.tensor(x, dtype=torch.float64, requires_grad=True)
    F = torch.nn.functional

    def situ(v, g, u):
        ag, au = F.linear(v, g), F.linear(v, u)
        return (B1 * torch.tanh(ag / B1) * torch.sigmoid(ag)) * (B2 * torch.tanh(au / B2))

    z = F.linear(xt, T["w_down"])
    s = torch.sigmoid(F.linear(xt, T["w_router"]))
    idt = torch.as_tensor(ids)
    sel = torch.gather(s, 1, idt)
    p = sel / sel.sum(1, keepdim=True)
    outs = torch.stack([F.linear(situ(z, T["w_g"][e], T["w_u"][e]), T["w_o"][e]) for e in range(6)], 1)
    u = sum(p[:, j:j + 1] * outs[torch.arange(x.shape[0]), idt[:, j]] for j in range(k))
    s_sh = sum(F.linear(situ(xt, T["sh_g"][j], T["sh_u"][j]), T["sh_o"][j]) for j in range(2))
    y = s_sh + F.linear(F.rms_norm(u, (u.shape[1],), T["rms_w"], eps=1e-6), T["w_up"])
    (y * torch.as_tensor(dy)).sum().backward()
    g = O.layer_backward(x, W, dy, ids=ids)
    np.testing.assert_allclose(g["x"], xt.grad.numpy(), rtol=1e-10, atol=1e-12)
    for n in ("w_down", "w_router", "w_up", "rms_w", "sh_g", "sh_u", "sh_o"):
        np.testing.assert_allclose(g[n], T[n].grad.numpy(), rtol=1e-10, atol=1e-12, err_msg=n)
    for e in range(6):
        for j, n in enumerate(("w_g", "w_u", "w_o")):
            np.testing.assert_allclose(g["routed"][e][j], T[n].grad[e].numpy(), rtol=1e-10, atol=1e-12)
