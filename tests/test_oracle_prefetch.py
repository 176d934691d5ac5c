"""Pins of the prefetch oracle ("Speculating Experts Accelerates Inference
for Mixture-of-Experts", items 1, 2 and 4): a hand-worked example, the
single-token case (the prefetched set is the predicted set, coverage is the
set intersection), optimality of the plan over all C-subsets on tiny inputs,
and conservation of picks between covered and missed experts."""

import itertools

import numpy as np
import pytest

from oracle import prefetch as pf


def test_hand_worked_example():
    # E = 6, two tokens, K = 3. Predicted counts: e2 x2, e5 x2, e0 x1, e4 x1.
    pred = np.array([[2, 5, 0], [5, 2, 4]])
    lst, nl, counts = pf.prefetch_plan(pred, 6, 3)
    assert counts.tolist() == [1, 0, 2, 0, 1, 2]
    assert lst.tolist() == [2, 5, 0] and nl == 3      # ties (2, 5) and (0, 4) to the lower index
    true = np.array([[2, 3, 0], [4, 5, 1]])
    covered, miss, nm = pf.prefetch_coverage(true, lst, 6)
    assert covered == 3                               # 2 and 0 (token 0), 5 (token 1); 3, 4, 1 not
    assert miss.tolist() == [1, 3, 4, -1, -1, -1] and nm == 3
    lst5, nl5, _ = pf.prefetch_plan(pred, 6, 5)
    assert lst5.tolist() == [2, 5, 0, 4, -1] and nl5 == 4


@pytest.mark.parametrize("seed", range(5))
def test_single_token_is_the_predicted_set(seed):
    rng = np.random.default_rng(seed)
    E, K = 64, 8
    pred = rng.choice(E, K, replace=False)[None, :]
    true = rng.choice(E, K, replace=False)[None, :]
    lst, nl, _ = pf.prefetch_plan(pred, E, K + 3)
    assert nl == K and sorted(lst[:K].tolist()) == lst[:K].tolist() == sorted(pred[0].tolist())
    assert (lst[K:] == -1).all()
    covered, miss, nm = pf.prefetch_coverage(true, lst, E)
    assert covered == len(set(pred[0]) & set(true[0]))
    assert miss[:nm].tolist() == sorted(set(true[0]) - set(pred[0]))


@pytest.mark.parametrize("seed", range(6))
def test_plan_is_the_best_c_subset(seed):
    rng = np.random.default_rng(seed + 10)
    E, n, K, C = 7, 5, 2, 3
    pred = np.stack([rng.choice(E, K, replace=False, p=np.arange(1, E + 1) / 28) for _ in range(n)])
    lst, nl, counts = pf.prefetch_plan(pred, E, C)
    named = [e for e in range(E) if counts[e] > 0]
    best = max(sum(counts[list(s)]) for s in itertools.combinations(named, min(C, len(named))))
    assert counts[lst[:nl]].sum() == best
    # order: counts non-increasing, equal counts by index
    keys = [(-counts[e], e) for e in lst[:nl]]
    assert keys == sorted(keys)
    # every listed count >= every unlisted named count
    rest = [counts[e] for e in named if e not in lst[:nl].tolist()]
    assert not rest or min(counts[lst[:nl]]) >= max(rest)


@pytest.mark.parametrize("C", [1, 4, 16, 64])
def test_covered_plus_missed_picks_conserve(C):
    rng = np.random.default_rng(C)
    E, n, K = 64, 40, 6
    pred = np.stack([rng.choice(E, K, replace=False) for _ in range(n)])
    true = np.stack([rng.choice(E, K, replace=False) for _ in range(n)])
    lst, nl, _ = pf.prefetch_plan(pred, E, C)
    covered, miss, nm = pf.prefetch_coverage(true, lst, E)
    missed_picks = sum(int((true == e).sum()) for e in miss[:nm])
    assert covered + missed_picks == n * K
    assert set(miss[:nm]).isdisjoint(set(lst[:nl]))
    assert (miss[nm:] == -1).all() and list(miss[:nm]) == sorted(miss[:nm])


def test_prediction_equal_to_truth_covers_everything():
    rng = np.random.default_rng(3)
    E, n, K = 32, 20, 4
    pred = np.stack([rng.choice(E, K, replace=False) for _ in range(n)])
    lst, nl, _ = pf.prefetch_plan(pred, E, E)
    covered, _, nm = pf.prefetch_coverage(pred, lst, E)
    assert covered == n * K and nm == 0


def test_out_of_range_picks_are_ignored():
    pred = np.array([[1, -1, 9], [1, 2, 8]])
    lst, nl, counts = pf.prefetch_plan(pred, 8, 4)
    assert counts.sum() == 3 and lst.tolist() == [1, 2, -1, -1]
    covered, miss, nm = pf.prefetch_coverage(np.array([[1, 8, -3]]), lst, 8)
    assert covered == 1 and nm == 0


def test_copy_moves_listed_experts_only():
    rng = np.random.default_rng(4)
    bank = rng.integers(0, 256, (5, 48), dtype=np.uint8)
    slots = rng.integers(0, 256, (3, 48), dtype=np.uint8)
    out = pf.prefetch_copy(bank, np.array([4, -1, 0]), slots)
    assert np.array_equal(out[0], bank[4]) and np.array_equal(out[2], bank[0])
    assert np.array_equal(out[1], slots[1])
