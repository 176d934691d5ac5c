"""Pins for moe_permute: bijection, counts, stability, row copies, and a
list-of-lists brute force; grouped source rows."""
import numpy as np
import pytest

from oracle import moe_permute, route_topk
from synth import to_bf16_bits


@pytest.mark.parametrize("N,E,K,H", [(1, 4, 2, 1), (50, 4, 2, 1), (333, 16, 6, 1), (200, 16, 8, 4)])
def test_invariants(N, E, K, H):
    rng = np.random.default_rng(N + E)
    idx, _ = route_topk(rng.standard_normal((N, E)), K, H)
    d = 8
    src = to_bf16_bits(rng.standard_normal((H, N, d)).astype(np.float32))
    r = moe_permute(idx, E, H, src)
    sop, pos, offs = r["slot_of_pair"], r["pair_of_slot"], r["expert_offsets"]
    assert np.array_equal(pos[sop], np.arange(N * K))
    assert np.array_equal(sop[pos], np.arange(N * K))
    assert offs[0] == 0 and offs[-1] == N * K and np.all(np.diff(offs) >= 0)
    flat = idx.reshape(-1)
    for e in range(E):
        seg = pos[offs[e]:offs[e + 1]]
        assert np.all(flat[seg] == e)
        assert np.all(np.diff(seg) > 0)          # stable: pair ids increase
    for p in range(N * K):
        i, k = divmod(p, K)
        assert np.array_equal(r["disp"][sop[p]], src[k // (K // H), i])


def test_against_lists():
    rng = np.random.default_rng(9)
    N, E, K = 40, 5, 3
    idx, _ = route_topk(rng.standard_normal((N, E)), K)
    r = moe_permute(idx, E)
    lists = [[] for _ in range(E)]
    for i in range(N):
        for k in range(K):
            lists[idx[i, k]].append(i * K + k)
    assert r["pair_of_slot"].tolist() == [p for l in lists for p in l]
    assert r["expert_offsets"].tolist() == [0] + list(np.cumsum([len(l) for l in lists]))


def test_empty():
    r = moe_permute(np.zeros((0, 2), dtype=np.int64), 4)
    assert r["expert_offsets"].tolist() == [0, 0, 0, 0, 0]
    assert len(r["slot_of_pair"]) == 0
