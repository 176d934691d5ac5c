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


def _predict_inputs(n, G, V, seed, fallback):
    rng = np.random.default_rng(seed)
    tok = rng.zipf(1.2, n).astype(np.int64) % V
    lut = rng.integers(0, G, V).astype(np.uint8)
    out = dict(tok=tok.astype(np.int32), lut=lut)
    if fallback:
        out.update(conf=rng.integers(0, 256, V).astype(np.uint8),
                   prev2=rng.integers(0, G, n).astype(np.uint8),
                   prev1=rng.integers(0, G, n).astype(np.uint8),
                   ngram=rng.integers(0, G, (G, G)).astype(np.uint8))
    return out


@pytest.mark.parametrize("n,G,fallback", [(64, 2, False), (4096, 4, False), (4096, 8, True),
                                          (4097, 4, True), (16384, 8, True), (1, 1, False),
                                          (3000, 256, True), (20000, 3, False)])
def test_predict_sort_against_oracle(n, G, fallback):
    """route_predict_sort on both sides of the one-workgroup limit: dest is
    the oracle's prediction and the maps are the oracle's stable shuffle of
    it, bit for bit."""
    a = _predict_inputs(n, G, 5000, n + G, fallback)
    fb = dict(conf=dev(a["conf"]), prev2=dev(a["prev2"]), prev1=dev(a["prev1"]),
              ngram=dev(a["ngram"])) if fallback else {}
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    dest, offs, ros, sor, rc = tr.route_predict_sort(dev(a["tok"]), dev(a["lut"]), G, err=err, **fb)
    sync()
    assert int(err.item()) == 0
    want = oracle.route_predict(a["tok"], a["lut"], a.get("conf"), a.get("prev2"), a.get("prev1"),
                                a.get("ngram"), 128, G=G)
    assert np.array_equal(host(dest), want)
    srs = oracle.srs_shuffle(np.zeros((1, n, 8), dtype=np.uint16), want, G)
    assert np.array_equal(host(offs), srs["offsets"])
    assert np.array_equal(host(ros), srs["row_of_src"])
    assert np.array_equal(host(sor), srs["src_of_row"])
    assert np.array_equal(host(rc), srs["row_cluster"])


@pytest.mark.parametrize("n", [3000, 9000])
def test_predict_sort_flags_like_predict_then_sort(n):
    """Tokens outside the vocabulary (cluster 0, TOKEN_RANGE), table entries
    past G and previous clusters past G (DEST_RANGE) come out as
    route_predict followed by srs_shuffle's sort: the same bytes and bits."""
    G, V = 4, 5000
    a = _predict_inputs(n, G, V, n, True)
    a["tok"][::97] = V + 5
    a["tok"][::131] = -3
    a["lut"][a["tok"][5]] = G + 2 if a["tok"][5] >= 0 else 0
    a["prev2"][7::211] = G
    a["conf"][:] = np.where(np.arange(V) % 3 == 0, 0, 255).astype(np.uint8)
    fb = dict(conf=dev(a["conf"]), prev2=dev(a["prev2"]), prev1=dev(a["prev1"]),
              ngram=dev(a["ngram"]))
    e1 = torch.zeros(1, dtype=torch.int32, device="cuda")
    dest, offs, ros, sor, rc = tr.route_predict_sort(dev(a["tok"]), dev(a["lut"]), G, err=e1, **fb)
    e2 = torch.zeros(1, dtype=torch.int32, device="cuda")
    d2 = tr.route_predict(dev(a["tok"]), dev(a["lut"]), G, err=e2, **fb)
    parts = torch.zeros((1, n, 8), dtype=torch.bfloat16, device="cuda")
    _, o2, r2, s2, c2 = tr.srs_shuffle(parts, d2, G, err=e2)
    sync()
    assert int(e1.item()) == int(e2.item())
    assert int(e1.item()) & tr.EBIT_TOKEN_RANGE and int(e1.item()) & tr.EBIT_DEST_RANGE
    assert torch.equal(dest, d2) and torch.equal(offs, o2) and torch.equal(ros, r2)
    valid = int(host(o2)[-1])
    assert torch.equal(sor[:valid], s2[:valid]) and torch.equal(rc[:valid], c2[:valid])
