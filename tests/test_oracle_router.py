"""Pins of the oracle's router (K3 sigmoid routing) against facts the pages
and the mathematics fix."""
import json
import math
import os

import numpy as np
import pytest

import oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _golden_case():
    g = json.load(open(os.path.join(GOLD, "router_closed_form.json")))
    w = np.zeros((g["n_routed"], g["hidden"]))
    for row, val in g["router_rows"].items():
        w[int(row)] = val
    x = np.full((g["tokens"], g["hidden"]), g["x_value"])
    return g, w, x


def test_closed_form_case_from_pages():
    g, w, x = _golden_case()
    r = O.route(x, w, np.zeros(g["n_routed"]), g["top_k"])
    assert set(r.ids.reshape(-1).tolist()) == set(g["expected_selected_set"])
    # every token picks expert 0 first (logit 32 > 16 > 0)
    assert (r.ids[:, 0] == 0).all() and (r.ids[:, 1] == 1).all()
    # p = (sigma(32), sigma(16)) / (sigma(32) + sigma(16)), written through tanh:
    # sigma(t) = (1 + tanh(t/2)) / 2
    s32, s16 = (1 + math.tanh(16.0)) / 2, (1 + math.tanh(8.0)) / 2
    np.testing.assert_allclose(r.p[0], [s32 / (s32 + s16), s16 / (s32 + s16)], rtol=0, atol=1e-15)
    np.testing.assert_allclose(r.p.sum(axis=1), 1.0, atol=1e-15)


def test_brute_force_topk_and_renorm():
    rng = np.random.default_rng(7)
    for R, k in [(5, 1), (8, 2), (16, 4), (13, 13)]:
        logits = rng.normal(size=(40, R)) * 2
        b = rng.uniform(-0.2, 0.2, size=R)
        r = O.route_from_logits(logits, b, k)
        for n in range(40):
            s = [1.0 / (1.0 + math.exp(-float(l))) for l in logits[n]]
            v = [s[i] + float(b[i]) for i in range(R)]
            top = sorted(range(R), key=lambda i: (-v[i], i))[:k]
            assert r.ids[n].tolist() == top
            tot = sum(s[i] for i in top)
            np.testing.assert_allclose(r.p[n], [s[i] / tot for i in top], rtol=1e-14)
            assert len(set(r.ids[n].tolist())) == k
            if k < R:
                assert r.margin[n] == pytest.approx(v[top[-1]] - sorted(v, reverse=True)[k], abs=1e-15)
            else:
                assert math.isinf(r.margin[n])


def test_bias_enters_selection_only():
    rng = np.random.default_rng(3)
    R, k = 10, 3
    logits = rng.normal(size=(30, R))
    forced = [7, 2, 9]
    b = np.zeros(R)
    b[forced] = 10.0
    r = O.route_from_logits(logits, b, k)
    s = 1.0 / (1.0 + np.exp(-logits))
    for n in range(30):
        assert set(r.ids[n].tolist()) == set(forced)
        sel = s[n, r.ids[n]]
        np.testing.assert_allclose(r.p[n], sel / sel.sum(), rtol=1e-15)
    # a bias that leaves every selection unchanged leaves p bit-identical
    r0 = O.route_from_logits(logits, np.zeros(R), k)
    tiny = np.full(R, 1e-3)  # uniform shift: same order everywhere
    r1 = O.route_from_logits(logits, tiny, k)
    np.testing.assert_array_equal(r0.ids, r1.ids)
    np.testing.assert_array_equal(r0.p, r1.p)


def test_all_equal_scores_tie_rule():
    R, k = 12, 5
    r = O.route(np.zeros((4, 6)), np.ones((R, 6)), np.zeros(R), k)
    assert (r.ids == np.arange(k)).all()
    np.testing.assert_array_equal(r.p, np.full((4, k), 1.0 / k))
    assert (r.margin == 0).all()


def test_k_equals_R_is_full_renormalised_mixture():
    rng = np.random.default_rng(11)
    logits = rng.normal(size=(6, 7))
    r = O.route_from_logits(logits, np.zeros(7), 7)
    s = 1 / (1 + np.exp(-logits))
    full = np.take_along_axis(s / s.sum(axis=1, keepdims=True), r.ids, axis=1)
    np.testing.assert_allclose(r.p, full, rtol=1e-14)


def test_sigmoid_matches_tanh_form_and_saturates():
    x = np.array([-800.0, -30.0, -1.0, 0.0, 1e-8, 2.5, 30.0, 800.0])
    ref = 0.5 * (1.0 + np.tanh(x / 2.0))  # loses relative accuracy for x << 0
    np.testing.assert_allclose(O.sigmoid(x), ref, rtol=1e-15, atol=4e-17)
    assert O.sigmoid(np.array([-800.0]))[0] == 0.0 and O.sigmoid(np.array([800.0]))[0] == 1.0
    # far tail: sigmoid(-30) = e^-30 / (1 + e^-30)
    assert O.sigmoid(np.array([-30.0]))[0] == pytest.approx(math.exp(-30) / (1 + math.exp(-30)), rel=1e-15)


def test_aux_and_z_loss_collapse_case():
    g, w, x = _golden_case()
    r = O.route(x, w, np.zeros(8), 2)
    aux, zl = O.balancing_losses(r.logits, r.ids, 8)
    assert aux > g["aux_collapsed_lower_bound"]
    assert zl > 0
    # closed form: f = (1/2, 1/2, 0...), P = s, so aux = 8 (s0 + s1) / 2;
    # lse = 32 + log(1 + e^-16 + 6 e^-32)
    s32, s16 = (1 + math.tanh(16.0)) / 2, (1 + math.tanh(8.0)) / 2
    assert aux == pytest.approx(8 * (s32 + s16) / 2, rel=1e-14)
    lse = 32 + math.log1p(math.exp(-16) + 6 * math.exp(-32))
    assert zl == pytest.approx(lse ** 2, rel=1e-14)
    rng = np.random.default_rng(0)
    xs = rng.normal(size=(64, 32))
    ws = rng.normal(size=(8, 32)) / math.sqrt(32)
    rs = O.route(xs, ws, np.zeros(8), 2)
    aux_spread, _ = O.balancing_losses(rs.logits, rs.ids, 8)
    assert aux > aux_spread


def test_softmax_topk_legacy_router():
    logits = np.array([[3.0, 1.0, 2.0, -1.0]])
    ids, p = O.route_softmax_topk(logits, 2)
    assert ids.tolist() == [[0, 2]]
    np.testing.assert_allclose(p[0], [1 / (1 + math.exp(-1)), math.exp(-1) / (1 + math.exp(-1))], rtol=1e-15)
