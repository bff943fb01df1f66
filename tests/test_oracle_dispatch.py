"""Pins of the oracle's permute-dispatch bookkeeping (brute force and invariants)."""
import numpy as np

import oracle as O


def _random_ids(rng, N, R, k):
    return np.stack([rng.permutation(R)[:k] for _ in range(N)]) if N else np.zeros((0, k), np.int64)


def test_brute_force_stable_sort():
    rng = np.random.default_rng(5)
    for N, R, k in [(1, 4, 1), (9, 5, 2), (33, 8, 3), (20, 6, 6)]:
        ids = _random_ids(rng, N, R, k)
        d = O.dispatch(ids, R)
        flat = ids.reshape(-1).tolist()
        want = sorted(range(N * k), key=lambda q: (flat[q], q))
        assert d.order.tolist() == want
        counts = [flat.count(e) for e in range(R)]
        assert d.counts.tolist() == counts
        assert d.offsets.tolist() == [sum(counts[:e]) for e in range(R)]
        assert d.capacity == max(counts)
        for pos, q in enumerate(want):
            e = flat[q]
            assert d.local_pos[pos] == pos - sum(counts[:e])
            assert 0 <= d.local_pos[pos] < counts[e]


def test_invariants_and_token_order_inside_expert():
    rng = np.random.default_rng(8)
    N, R, k = 200, 16, 4
    ids = _random_ids(rng, N, R, k)
    d = O.dispatch(ids, R)
    assert d.counts.sum() == N * k
    assert sorted(d.order.tolist()) == list(range(N * k))
    for e in range(R):
        seg = d.order[d.offsets[e]:d.offsets[e] + d.counts[e]]
        toks = seg // k
        assert (np.diff(toks) > 0).all()  # ids of one token are distinct -> strictly ascending
        assert (ids.reshape(-1)[seg] == e).all()


def test_k_equals_R_and_empty():
    N, R = 7, 5
    ids = np.tile(np.arange(R), (N, 1))
    d = O.dispatch(ids, R)
    assert (d.counts == N).all() and d.capacity == N
    d0 = O.dispatch(np.zeros((0, 2), np.int64), R)
    assert d0.capacity == 0 and d0.counts.sum() == 0


def test_padded_layout_rows():
    rng = np.random.default_rng(2)
    N, R, k, ell = 25, 6, 2, 3
    ids = _random_ids(rng, N, R, k)
    z = rng.normal(size=(N, ell))
    d = O.dispatch(ids, R)
    pad = O.padded_layout(z, ids, R, d)
    assert pad.shape == (R, d.capacity, ell)
    for e in range(R):
        toks = [n for n in range(N) if e in ids[n].tolist()]
        np.testing.assert_array_equal(pad[e, :len(toks)], z[toks])
        assert (pad[e, len(toks):] == 0).all()
