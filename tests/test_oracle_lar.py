"""Pins for lar_count: the locality formulas rho_moe = 1/G and
rho_foe = min(H/G, 1) under uniform routing (golden fixture from the FoE
article), all-local and none-local constructions, and a Python loop."""
import os

import numpy as np
import pytest

from oracle import lar_count, route_topk
from synth import default_expert_cluster, foe_row_cluster

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "locality_rho.txt")


def _rows():
    out = []
    for line in open(GOLDEN):
        line = line.split("#")[0].strip()
        if line:
            G, H, rm, rf = line.split()
            out.append((int(G), int(H), float(rm), float(rf)))
    return out


def _within(count, trials, p):
    sigma = np.sqrt(trials * p * (1 - p))
    return abs(count - trials * p) <= 4 * sigma + 1e-9


@pytest.mark.parametrize("G,H,rho_moe,rho_foe", _rows())
def test_uniform_routing_locality(G, H, rho_moe, rho_foe):
    rng = np.random.default_rng(G * 100 + H)
    N, E = 20000, 16 * max(G, H)
    # plain MoE: token rows on uniform random clusters
    K = 2
    idx, _ = route_topk(rng.standard_normal((N, E)), K)
    rc = rng.integers(0, G, N)
    local = lar_count(idx, K, 1, rc, default_expert_cluster(E, G))
    assert _within(local, N * K, rho_moe)
    # FoE: group h's copy of token i on cluster foe_row_cluster
    K = 2 * H
    idx, _ = route_topk(rng.standard_normal((N, E)), K, H)
    local = lar_count(idx, K, H, foe_row_cluster(N, H, G), default_expert_cluster(E, G))
    assert _within(local, N * K, min(rho_foe, 1.0 - 1e-12)) or (rho_foe == 1.0 and local == N * K)


def test_all_local_and_none_local():
    N, E, G, K = 300, 12, 3, 2
    ec = default_expert_cluster(E, G)
    rng = np.random.default_rng(1)
    rc = rng.integers(0, G, N)
    logits = rng.standard_normal((N, E))
    # push the row's own cluster's experts to the top
    logits[ec[None, :] == rc[:, None]] += 100.0
    idx, _ = route_topk(logits, K)
    assert lar_count(idx, K, 1, rc, ec) == N * K
    assert lar_count(idx, K, 1, (rc + 1) % G, ec) == 0


def test_against_loop():
    rng = np.random.default_rng(2)
    N, E, H, K, G = 97, 16, 2, 4, 4
    idx, _ = route_topk(rng.standard_normal((N, E)), K, H)
    rc = rng.integers(0, G, N * H)
    ec = rng.integers(0, G, E)
    n = 0
    for i in range(N):
        for k in range(K):
            h = k // (K // H)
            n += int(ec[idx[i, k]] == rc[i * H + h])
    assert lar_count(idx, K, H, rc, ec) == n
