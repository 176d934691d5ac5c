"""Pins for srs_shuffle: bucket-loop brute force, P=1 permutation, G=1
reduce, P=2 exact rational rounding, exact-sum rounding for P=4."""
from fractions import Fraction

import numpy as np
import pytest

from oracle import srs_shuffle
from oracle.bf16 import bf16_to_f64
from synth import to_bf16_bits


def _parts(P, N, d, seed):
    rng = np.random.default_rng(seed)
    return to_bf16_bits(rng.standard_normal((P, N, d)).astype(np.float32))


def _nearest_even(x: Fraction) -> int:
    """bf16 bits nearest to the exact rational x (normal range), ties to even."""
    f = float(x)
    base = int(np.float32(f).view(np.uint32) >> 16)
    best = None
    for b in range(base - 2, base + 3):
        v = Fraction(float(bf16_to_f64(np.array([b & 0xFFFF], dtype=np.uint16))[0]))
        key = (abs(v - x), b & 1)
        if best is None or key < best[0]:
            best = (key, b & 0xFFFF)
    return best[1]


def test_bucket_loop():
    P, N, d, G = 2, 300, 16, 5
    parts = _parts(P, N, d, 1)
    dest = np.random.default_rng(2).integers(0, G, N)
    r = srs_shuffle(parts, dest, G)
    buckets = [[] for _ in range(G)]
    for i in range(N):
        buckets[dest[i]].append(i)
    order = [i for b in buckets for i in b]
    assert r["src_of_row"].tolist() == order
    offs = [0]
    for b in buckets:
        offs.append(offs[-1] + len(b))
    assert r["offsets"].tolist() == offs
    for row, i in enumerate(order):
        assert r["row_of_src"][i] == row
        assert r["row_cluster"][row] == dest[i]
        assert np.array_equal(r["out"][row], r["reduced"][i])


def test_single_partial_is_pure_permutation():
    parts = _parts(1, 200, 8, 3)
    dest = np.random.default_rng(4).integers(0, 7, 200)
    r = srs_shuffle(parts, dest, 7)
    assert np.array_equal(r["out"], parts[0][r["src_of_row"]])


def test_single_cluster_is_pure_reduce():
    parts = _parts(3, 64, 24, 5)
    r = srs_shuffle(parts, None, 1)
    assert np.array_equal(r["src_of_row"], np.arange(64))
    assert r["offsets"].tolist() == [0, 64]
    assert np.array_equal(r["out"], r["reduced"])


def test_two_partials_round_the_exact_sum_once():
    parts = _parts(2, 40, 32, 6)
    r = srs_shuffle(parts, None, 1)
    a = bf16_to_f64(parts[0]).ravel()
    b = bf16_to_f64(parts[1]).ravel()
    out = r["out"].ravel()
    for j in range(len(a)):
        s = Fraction(a[j]) + Fraction(b[j])
        if s == 0:
            assert out[j] & 0x7FFF == 0
            continue
        assert out[j] == _nearest_even(s), j


def test_four_partials_exact_sums():
    # small multiples of 2^-4 keep every partial sum exact in binary32, so the
    # result must be the nearest bf16 of the exact total
    rng = np.random.default_rng(11)
    vals = rng.integers(-2000, 2000, (4, 30, 16)) / 16.0
    parts = to_bf16_bits(vals.astype(np.float32))
    dec = bf16_to_f64(parts)
    r = srs_shuffle(parts, None, 1)
    tot = dec.sum(axis=0).ravel()
    out = r["out"].ravel()
    for j in range(len(tot)):
        if tot[j] == 0:
            assert out[j] & 0x7FFF == 0
        else:
            assert out[j] == _nearest_even(Fraction(tot[j]))


def test_bad_dest_raises():
    parts = _parts(1, 10, 8, 0)
    with pytest.raises(ValueError):
        srs_shuffle(parts, np.full(10, 3), 3)


def test_signed_zero_sum_is_ieee_fold():
    # -0 + -0 = -0 under IEEE addition; the sum starts at the first partial
    parts = np.full((2, 1, 8), 0x8000, dtype=np.uint16)
    assert np.all(srs_shuffle(parts, None, 1)["out"] == 0x8000)
    parts[1] = 0x0000
    assert np.all(srs_shuffle(parts, None, 1)["out"] == 0x0000)
