"""Pins of the s-EG oracle ("Speculative MoE" notes, sections 3.2 and 4.2).

Each test checks the oracle against something other than its own formulas:
the published outputs of the reference SplitMix64 generator, invariants the
definitions imply (capacity, conservation, bounds, relabelling), closed forms
of the objective, and a planted profile whose optimal placement is known.
"""

import math

import numpy as np
import pytest

from oracle import eg


# ------------------------------------------------------------- random numbers
def test_splitmix64_reference_outputs():
    # first three outputs of the reference SplitMix64 generator seeded with 0
    assert [eg.splitmix64(0, n) for n in (1, 2, 3)] == [
        0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]


def test_uniform01_range_and_moments():
    u = np.array([eg.uniform01(77, n) for n in range(1, 20001)])
    assert u.min() >= 0.0 and u.max() < 1.0
    assert abs(u.mean() - 0.5) < 0.01
    assert abs(u.var() - 1.0 / 12.0) < 0.005


# -------------------------------------------------------------------- profile
def _planted(U=40, E=16, G=4, K=2, n=600, seed=3):
    """Tokens whose experts all sit in one planted group (a placement exists
    with every activation local)."""
    rng = np.random.default_rng(seed)
    groups = rng.permutation(E).reshape(G, E // G)       # planted placement
    planted = np.empty(E, dtype=np.uint8)
    for g in range(G):
        planted[groups[g]] = g
    home = rng.integers(0, G, U)
    tok = rng.integers(0, U, n)
    idx = np.stack([rng.choice(groups[home[t]], K, replace=False) for t in tok])
    return tok, idx, planted


def test_profile_conservation():
    tok, idx, _ = _planted()
    counts, freq = eg.coact_profile(tok, idx, np.arange(40), 40, 16)
    assert counts.sum() == idx.size and freq.sum() == len(tok)
    assert np.array_equal(counts.sum(axis=1), 2 * freq)
    with pytest.raises(ValueError):
        eg.coact_profile(tok, idx, np.full(40, -1), 40, 16)


# ---------------------------------------------------------------------- score
def test_score_single_cluster_and_bounds():
    rng = np.random.default_rng(5)
    counts = rng.integers(0, 9, (30, 12))
    freq = rng.integers(1, 5, 30)
    T, F = counts.sum(), freq.sum()
    local, load = eg.eg_score(counts, freq, np.zeros((1, 12), np.uint8), 1)
    assert local[0] == T and load[0, 0] == F
    place = np.stack([rng.permutation(np.repeat(np.arange(3), 4)) for _ in range(20)])
    local, load = eg.eg_score(counts, freq, place, 3)
    # the best of G partial sums is at least their mean and at most their total
    assert (local <= T).all() and (3 * local >= T).all()
    assert (load.sum(axis=1) == F).all()


def test_score_relabelling():
    rng = np.random.default_rng(6)
    counts = rng.integers(0, 9, (25, 8))
    freq = rng.integers(1, 4, 25)
    p = rng.permutation(np.repeat(np.arange(4), 2))
    relabel = np.array([2, 0, 3, 1])
    l1, d1 = eg.eg_score(counts, freq, p[None], 4)
    l2, d2 = eg.eg_score(counts, freq, relabel[p][None], 4)
    # the best share of every token does not depend on the labels (its loads
    # may, where the lowest-label tie rule picks a different cluster)
    assert l1[0] == l2[0]
    assert d1.sum() == d2.sum() == freq.sum()


def test_score_planted_is_all_local():
    tok, idx, planted = _planted()
    counts, freq = eg.coact_profile(tok, idx, np.arange(40), 40, 16)
    local, _ = eg.eg_score(counts, freq, planted[None], 4)
    assert local[0] == counts.sum()


def test_objective_closed_forms():
    # all local and perfectly balanced -> 0; nothing local, one cluster full
    J = eg.eg_objective([100, 0], [[25, 25, 25, 25], [100, 0, 0, 0]], 100, 100, 4, 0.5)
    assert J[0] == 0.0
    assert J[1] == pytest.approx(0.5 * 1.0 + 0.5 * 3.0)


# --------------------------------------------------------------------- sample
def test_sample_capacity():
    rng = np.random.default_rng(8)
    P = rng.random((24, 4))
    P /= P.sum(axis=1, keepdims=True)
    place = eg.eg_sample(P, 16, 4, 11, 0)
    for b in range(16):
        assert (np.bincount(place[b], minlength=4) == 6).all()


def test_sample_reproduces_a_certain_table():
    rng = np.random.default_rng(9)
    x0 = rng.permutation(np.repeat(np.arange(4), 5)).astype(np.uint8)
    P = np.zeros((20, 4))
    P[np.arange(20), x0] = 1.0
    place = eg.eg_sample(P, 8, 4, 5, 3)
    assert (place == x0[None]).all()


def test_sample_first_expert_follows_p():
    P = np.full((8, 2), 0.5)
    P[0] = [0.25, 0.75]
    place = eg.eg_sample(P, 4000, 2, 21, 0)
    frac = (place[:, 0] == 1).mean()
    assert abs(frac - 0.75) < 0.03   # about 4.4 standard errors


# --------------------------------------------------------------------- update
def test_update_single_elite_full_step():
    place = np.array([[0, 1, 1, 0], [1, 0, 0, 1], [0, 0, 1, 1]], np.uint8)
    J = np.array([0.3, 0.1, 0.2])
    P = np.full((4, 2), 0.5)
    Pn, bJ, bp = eg.eg_update(P, place, J, 1, 1.0, np.inf, np.zeros(4, np.uint8))
    assert np.array_equal(Pn, np.eye(2)[place[1]])
    assert bJ == 0.1 and np.array_equal(bp, place[1])
    # no strict improvement keeps the incumbent
    Pn, bJ2, bp2 = eg.eg_update(P, place, J, 1, 1.0, 0.1, place[0])
    assert bJ2 == 0.1 and np.array_equal(bp2, place[0])


def test_update_ties_go_to_lower_index_and_mix():
    place = np.array([[0, 1], [1, 0], [0, 1]], np.uint8)
    J = np.array([0.5, 0.2, 0.2])
    P = np.full((2, 2), 0.5)
    Pn, bJ, bp = eg.eg_update(P, place, J, 1, 0.5, np.inf, np.zeros(2, np.uint8))
    assert np.array_equal(bp, place[1])
    assert np.allclose(Pn, 0.5 * np.eye(2)[place[1]] + 0.25)


# ------------------------------------------------------------ the whole solve
def test_ceo_finds_the_planted_optimum():
    tok, idx, planted = _planted()
    counts, freq = eg.coact_profile(tok, idx, np.arange(40), 40, 16)
    best, J, P, hist = eg.ceo_place(counts, freq, 4, theta=0.0, B=64, iters=25, rho=0.1,
                                    alpha=0.7, seed=1)
    local, _ = eg.eg_score(counts, freq, best[None], 4)
    assert local[0] == counts.sum() and J == 0.0
    assert all(a >= b for a, b in zip(hist, hist[1:]))   # best never gets worse
    assert math.isclose(P.sum(), 16.0)                    # rows stay distributions
