"""Pins of the oracle's router top-k and weights."""
import math

import numpy as np
import scipy.special

from oracle import route


def test_brute_force_sort_and_softmax():
    rng = np.random.default_rng(1)
    for _ in range(200):
        M, E = int(rng.integers(1, 5)), int(rng.integers(2, 20))
        k = int(rng.integers(1, E + 1))
        z = rng.standard_normal((M, E)).astype(np.float32)
        if rng.random() < 0.5:   # plant exact ties
            z = np.round(z * 2) / 2
        ids, w = route(z, k)
        for m in range(M):
            order = np.lexsort((np.arange(E), -z[m].astype(np.float64)))   # logit desc, id asc
            assert list(ids[m]) == list(order[:k])
            ref = scipy.special.softmax(z[m, order[:k]].astype(np.float64))
            np.testing.assert_allclose(w[m], ref, rtol=1e-14, atol=0)
            assert abs(w[m].sum() - 1.0) < 1e-14


def test_k_equals_e_is_the_full_softmax():
    rng = np.random.default_rng(2)
    z = rng.standard_normal((3, 16)).astype(np.float32)
    ids, w = route(z, 16)
    for m in range(3):
        full = scipy.special.softmax(z[m].astype(np.float64))
        np.testing.assert_allclose(w[m], full[ids[m]], rtol=1e-14)
        assert sorted(ids[m]) == list(range(16))


def test_ties_break_to_the_lower_expert_id():
    z = np.zeros((1, 10), dtype=np.float32)
    ids, w = route(z, 4)
    assert list(ids[0]) == [0, 1, 2, 3]
    assert np.all(w == 0.25)
    z = np.array([[1.0, 2.0, 2.0, -0.0, 0.0, 2.0]], dtype=np.float32)
    ids, _ = route(z, 6)
    assert list(ids[0]) == [1, 2, 5, 0, 3, 4]   # -0 and +0 tie, lower id first
    for a, b in ((0.0, -0.0), (-0.0, 0.0)):
        ids, w = route(np.array([[a, b, -1.0]], dtype=np.float32), 1)
        assert ids[0, 0] == 0 and w[0, 0] == 1.0


def test_non_finite_logits():
    z = np.array([[np.nan, -np.inf, 0.5, np.nan, -np.inf]], dtype=np.float32)
    ids, w = route(z, 4)
    assert list(ids[0]) == [2, 1, 4, 0]       # NaN sorts below -inf
    assert list(w[0]) == [1.0, 0.0, 0.0, 0.0]
    z = np.array([[np.inf, 1.0, np.inf, 3.0]], dtype=np.float32)
    ids, w = route(z, 3)
    assert list(ids[0]) == [0, 2, 3] and list(w[0]) == [0.5, 0.5, 0.0]
    z = np.array([[-np.inf, -np.inf, np.nan]], dtype=np.float32)
    ids, w = route(z, 2)
    assert list(ids[0]) == [0, 1] and list(w[0]) == [0.5, 0.5]
