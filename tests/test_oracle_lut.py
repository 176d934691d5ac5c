"""Pins for the offline table builder: per-id brute force over shares,
ties to the lower cluster, and the confidence byte."""
import numpy as np

from oracle import route_lut_build, route_topk


def test_bruteforce_and_ties():
    rng = np.random.default_rng(0)
    n, E, K, G, V = 200, 16, 4, 4, 1000
    ids = rng.choice(V, n, replace=False)
    idx, w = route_topk(rng.standard_normal((n, E)), K)
    ec = (np.arange(E) // (E // G)).astype(np.uint8)
    lut = np.zeros(V, dtype=np.uint8)
    conf = np.zeros(V, dtype=np.uint8)
    route_lut_build(ids, idx, w.astype(np.float32), ec, G, lut, conf)
    for i in range(n):
        share = {c: 0.0 for c in range(G)}
        for k in range(K):
            share[int(ec[idx[i, k]])] += float(np.float32(w[i, k]))
        best = max(share.values())
        c = min(c for c in range(G) if abs(share[c] - best) < 1e-6)
        assert lut[ids[i]] == c
        assert abs(int(conf[ids[i]]) - 255 * best) <= 0.5 + 1e-3


def test_exact_tie_goes_to_lower_cluster():
    ec = np.array([0, 0, 1, 1], dtype=np.uint8)
    idx = np.array([[2, 0]])
    w = np.array([[0.5, 0.5]], dtype=np.float32)
    lut = np.full(4, 9, dtype=np.uint8)
    conf = np.zeros(4, dtype=np.uint8)
    route_lut_build(np.array([3]), idx, w, ec, 2, lut, conf)
    assert lut[3] == 0 and conf[3] == 128   # 127.5 + 0.5 -> 128
    w = np.array([[1.0, 0.0]], dtype=np.float32)
    route_lut_build(np.array([1]), idx, w, ec, 2, lut, conf)
    assert lut[1] == 1 and conf[1] == 255
