"""GPU parity of the counting sort behind srs_shuffle and moe_permute on both
sides of the switch between its one-workgroup form (up to 16384 keys and
256 bins) and its two-launch form: offsets, forward and inverse maps and
keys bit-exact against the oracle's stable sort, with skewed, single-bin
and out-of-range keys."""
import numpy as np
import pytest
import torch

import oracle
import token_routing_speculation_amd as tr
from tests.gpu_helpers import dev, host, sync

pytestmark = pytest.mark.gpu


def _skewed(n, B, seed):
    """Zipf-like keys: a few bins hold most of them, many bins stay empty."""
    rng = np.random.default_rng(seed)
    k = np.minimum(rng.zipf(1.3, n) - 1, B - 1)
    return rng.permutation(B)[k]


@pytest.mark.parametrize("n,G", [(16384, 8), (16385, 8), (16384, 256), (16385, 256),
                                 (1, 1), (65, 2), (16000, 3), (20000, 5)])
@pytest.mark.parametrize("skew", [False, True])
def test_shuffle_sort_both_forms(n, G, skew):
    rng = np.random.default_rng(n + G)
    dest = (_skewed(n, G, n) if skew else rng.integers(0, G, n)).astype(np.uint8)
    parts = rng.integers(0, 1 << 16, (1, n, 8), dtype=np.int64).astype(np.uint16)
    parts &= 0xbfff                  # finite bf16 values only
    want = oracle.srs_shuffle(parts, dest.astype(np.int64), G)
    out, offs, ros, sor, rc = tr.srs_shuffle(dev(parts), dev(dest), G)
    assert np.array_equal(host(offs), want["offsets"])
    assert np.array_equal(host(ros), want["row_of_src"])
    assert np.array_equal(host(sor), want["src_of_row"])
    assert np.array_equal(host(rc), want["row_cluster"])
    assert np.array_equal(host(out), want["out"])


@pytest.mark.parametrize("n,K,E", [(8192, 2, 8), (8193, 2, 8), (2048, 8, 256), (2049, 8, 256),
                                   (4096, 4, 257), (1, 1, 1), (5461, 3, 160)])
def test_permute_sort_both_forms(n, K, E):
    rng = np.random.default_rng(n * K + E)
    idx = np.stack([rng.permutation(E)[:K] if E >= K else rng.integers(0, E, K)
                    for _ in range(n)]).astype(np.int32)
    want = oracle.moe_permute(idx, E)
    offs, sop, pos, _ = tr.moe_permute(dev(idx), E)
    assert np.array_equal(host(offs), want["expert_offsets"])
    assert np.array_equal(host(sop), want["slot_of_pair"])
    assert np.array_equal(host(pos), want["pair_of_slot"])


@pytest.mark.parametrize("n", [5000, 20000])
def test_sort_flags_out_of_range_keys(n):
    """Keys past the bin count (and negative expert ids) are flagged and get
    position -1, in both forms; the rest sort as if they were absent."""
    E, K = 16, 1
    rng = np.random.default_rng(n)
    idx = rng.integers(0, E, (n, K)).astype(np.int32)
    bad = rng.choice(n, 7, replace=False)
    idx[bad[:4], 0] = E + 3
    idx[bad[4:], 0] = -2
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    offs, sop, pos, _ = tr.moe_permute(dev(idx), E, err=err)
    sync()
    assert int(err.item()) & tr.EBIT_EXPERT_RANGE
    s = host(sop)
    assert np.all(s[bad] == -1)
    good = np.setdiff1d(np.arange(n), bad)
    ref = oracle.moe_permute(idx[good], E)
    assert np.array_equal(host(offs), ref["expert_offsets"])
    assert np.array_equal(s[good], ref["slot_of_pair"])
    assert np.array_equal(host(pos)[: n - 7], good[ref["pair_of_slot"]])
