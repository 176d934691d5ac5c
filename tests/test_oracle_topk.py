"""Pins for route_topk: all-subsets brute force, grouped = per-slice plain,
K = E permutation, planted ties and signed zeros, scipy softmax weights."""
import itertools

import numpy as np
import pytest
from scipy.special import softmax

from oracle import route_topk


def _key(v, e):
    return (0.0 if v == 0 else float(v), -e)


def _brute_topk(row, K):
    """The unique K-subset whose every key beats every key outside it."""
    E = len(row)
    keys = [_key(row[e], e) for e in range(E)]
    found = []
    for S in itertools.combinations(range(E), K):
        rest = [e for e in range(E) if e not in S]
        if not rest or min(keys[s] for s in S) > max(keys[u] for u in rest):
            found.append(S)
    assert len(found) == 1
    return sorted(found[0], key=lambda e: keys[e], reverse=True)


@pytest.mark.parametrize("E,K", [(4, 1), (4, 2), (6, 3), (7, 4), (5, 5)])
def test_brute_force_small(E, K):
    rng = np.random.default_rng(E * 10 + K)
    # few distinct values so ties are common
    logits = rng.integers(-3, 4, (200, E)).astype(np.float32)
    logits[rng.random((200, E)) < 0.1] = -0.0
    idx, _ = route_topk(logits, K)
    for i in range(200):
        assert idx[i].tolist() == _brute_topk(logits[i], K)


@pytest.mark.parametrize("E,H,K", [(8, 2, 4), (12, 3, 6), (16, 4, 8), (6, 6, 6)])
def test_grouped_is_plain_per_group(E, H, K):
    rng = np.random.default_rng(E + H)
    logits = rng.integers(-2, 3, (150, E)).astype(np.float32)
    idx, w = route_topk(logits, K, H)
    eg, kg = E // H, K // H
    for i in range(150):
        for h in range(H):
            want = [e + h * eg for e in _brute_topk(logits[i, h * eg:(h + 1) * eg], kg)]
            assert idx[i, h * kg:(h + 1) * kg].tolist() == want
    # renorm=1: every group's weights sum to 1
    assert np.allclose(w.reshape(150, H, kg).sum(axis=2), 1.0, atol=1e-14)


def test_grouped_with_one_group_equals_plain():
    logits = np.random.default_rng(5).standard_normal((100, 32))
    a = route_topk(logits, 6, 1)
    idx = np.argsort(-logits, axis=1, kind="stable")[:, :6]
    assert np.array_equal(a[0], idx)


def test_k_equals_e_is_sorted_permutation():
    logits = np.random.default_rng(6).standard_normal((50, 9))
    idx, w = route_topk(logits, 9)
    for i in range(50):
        assert sorted(idx[i].tolist()) == list(range(9))
        assert np.all(np.diff(logits[i, idx[i]]) <= 0)
    idx0, w0 = route_topk(logits, 9, renorm=0)
    assert np.allclose(w0, np.take_along_axis(softmax(logits, axis=1), idx0, axis=1), rtol=1e-13)


def test_planted_ties_and_signed_zero():
    logits = np.array([[1.0, 3.0, 3.0, 2.0],
                       [-0.0, 0.0, -1.0, -1.0],
                       [0.0, -0.0, -2.0, 5.0],
                       [7.0, 7.0, 7.0, 7.0]])
    idx, _ = route_topk(logits, 2)
    assert idx.tolist() == [[1, 2], [0, 1], [3, 0], [0, 1]]


def test_weights_against_scipy_softmax():
    rng = np.random.default_rng(7)
    logits = rng.standard_normal((80, 20)) * 3
    idx, w1 = route_topk(logits, 5, renorm=1)
    sel = np.take_along_axis(logits, idx, axis=1)
    assert np.allclose(w1, softmax(sel, axis=1), rtol=1e-13)
    idx0, w0 = route_topk(logits, 5, renorm=0)
    full = softmax(logits, axis=1)
    assert np.allclose(w0, np.take_along_axis(full, idx0, axis=1), rtol=1e-13)
    assert np.all(w0.sum(axis=1) < 1.0)


def test_bad_shapes_raise():
    with pytest.raises(ValueError):
        route_topk(np.zeros((2, 6)), 4, 4)      # E % H != 0
    with pytest.raises(ValueError):
        route_topk(np.zeros((2, 8)), 10, 2)     # K/H = 5 > E/H = 4
    with pytest.raises(ValueError):
        route_topk(np.zeros((2, 8)), 3, 2)      # K % H != 0
