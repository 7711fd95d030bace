"""Pins of the oracle's routing and permutation: brute force with Python's
sort, the full softmax (scipy) restricted and renormalised, and invariants."""
import numpy as np
import pytest
import scipy.special

from oracle import moe


def _brute_route(l, k):
    T, E = l.shape
    ids = np.zeros((T, k), np.int64)
    for t in range(T):
        order = sorted(range(E), key=lambda e: (-float(l[t, e]), e))
        ids[t] = order[:k]
    return ids


@pytest.mark.parametrize("T,E,k", [(1, 1, 1), (5, 8, 2), (33, 64, 6), (17, 256, 8), (4, 384, 8), (3, 9, 9)])
def test_route_brute_force(T, E, k):
    rng = np.random.default_rng(T * 1000 + E)
    l = rng.standard_normal((T, E)).astype(np.float32)
    ids, w = moe.route(l, k)
    assert np.array_equal(ids, _brute_route(l, k))
    # weights: softmax over ALL experts, restricted to the picks, renormalised
    full = scipy.special.softmax(l.astype(np.float64), axis=1)
    sel = np.take_along_axis(full, ids.astype(np.int64), axis=1)
    assert np.allclose(w, sel / sel.sum(axis=1, keepdims=True), rtol=1e-13, atol=1e-15)


def test_route_invariants():
    rng = np.random.default_rng(2)
    l = (rng.standard_normal((200, 64)) * 3).astype(np.float32)
    ids, w = moe.route(l, 6)
    assert np.allclose(w.sum(axis=1), 1.0, atol=1e-12)
    assert np.all(np.diff(w, axis=1) <= 0)
    assert all(len(set(r)) == 6 for r in ids.tolist())


def test_route_k_equals_E_is_full_softmax():
    rng = np.random.default_rng(4)
    l = rng.standard_normal((10, 12)).astype(np.float32)
    ids, w = moe.route(l, 12)
    full = scipy.special.softmax(l.astype(np.float64), axis=1)
    back = np.zeros_like(full)
    np.put_along_axis(back, ids.astype(np.int64), w, axis=1)
    assert np.allclose(back, full, rtol=1e-13)


def test_route_ties_go_to_lower_id_and_signed_zero_ties():
    l = np.array([[1.0, 3.0, 3.0, 0.0, -0.0, 3.0],
                  [-0.0, 0.0, -1.0, 0.0, -0.0, -2.0]], np.float32)
    ids, w = moe.route(l, 4)
    assert ids[0].tolist() == [1, 2, 5, 0]
    assert ids[1].tolist() == [0, 1, 3, 4]
    assert np.allclose(w[1], 0.25)


def test_route_rejects_nonfinite():
    with pytest.raises(ValueError):
        moe.route(np.array([[np.nan, 1.0]], np.float32), 1)


@pytest.mark.parametrize("T,E,k", [(1, 1, 1), (16, 8, 2), (64, 64, 6), (300, 256, 8), (7, 1024, 3)])
def test_permute_brute_force(T, E, k):
    rng = np.random.default_rng(T + E)
    ids, _ = moe.route(rng.standard_normal((T, E)).astype(np.float32), k)
    offsets, sp, pp = moe.permute(ids, E)
    flat = ids.ravel().tolist()
    want = sorted(range(len(flat)), key=lambda p: (flat[p], p))
    assert sp.tolist() == want
    counts = [flat.count(e) for e in range(E)]
    assert offsets.tolist() == [sum(counts[:e]) for e in range(E + 1)]
    assert np.array_equal(pp[sp], np.arange(len(flat)))
    assert np.array_equal(sp[pp], np.arange(len(flat)))
    for e in range(E):
        assert all(flat[p] == e for p in sp[offsets[e]:offsets[e + 1]])


def test_permute_rejects_out_of_range():
    with pytest.raises(ValueError):
        moe.permute(np.array([[0, 8]]), 8)
