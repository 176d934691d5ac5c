"""GPU parity of srs_shuffle_route (the shuffled reduce, then the router,
top-K and local activation count of every reduced row, one kernel after the
sort): every shuffle output bit-exact against the oracle's shuffle; the
logits against the oracle's gate on the oracle's reduced rows; the top-K
indices bit-exact against the oracle's top-K of the logits the kernel wrote
(the ranking is decided in binary32 on both sides), the weights within 1e-5
of the oracle's softmax of them; the count exactly the oracle's LAR of those
picks."""
import numpy as np
import pytest
import torch

import oracle
import token_routing_speculation_amd as tr
from synth import to_bf16_bits
from tests.gpu_helpers import dev, host, assert_rel, assert_dot_bound, sync

pytestmark = pytest.mark.gpu

LOGIT_TOL = 1e-2      # the gate's stated bar (max relative error, row-rms floored)
F32_TOL = 1e-4        # binary32 accumulation of exact bf16 products


def _bf16(shape, seed, scale=1.0):
    return to_bf16_bits((np.random.default_rng(seed).standard_normal(shape) * scale).astype(np.float32))


def _inputs(n, d, P, G, E):
    rng = np.random.default_rng(n * 3 + d + E)
    parts = _bf16((P, n, d), n * 7 + d + P)
    dest = rng.integers(0, G, n, dtype=np.int64).astype(np.uint8)
    w = _bf16((E, d), E + d, 1 / np.sqrt(d))
    ec = rng.integers(0, G, E, dtype=np.int64).astype(np.uint8)
    return parts, dest, w, ec


def _run(parts, dest, G, w, K, ec, renorm=1, **kw):
    local = torch.zeros(1, dtype=torch.int64, device="cuda")
    r = tr.srs_shuffle_route(dev(parts), None if dest is None else dev(dest), G, dev(w), K,
                             renorm=renorm, expert_cluster=None if ec is None else dev(ec),
                             local=None if ec is None else local, **kw)
    sync()
    return r, local


def _check(parts, dest, G, w, K, ec, renorm, got, local):
    out, offs, ros, sor, rc, lg, idx, wt = got
    want = oracle.srs_shuffle(parts, None if dest is None else dest.astype(np.int64), G)
    assert np.array_equal(host(offs), want["offsets"])
    assert np.array_equal(host(ros), want["row_of_src"])
    assert np.array_equal(host(sor), want["src_of_row"])
    assert np.array_equal(host(rc), want["row_cluster"])
    assert np.array_equal(host(out), want["out"])
    ref = oracle.route_gate(want["out"], w)
    lgh = host(lg)
    assert_rel(lgh, ref, LOGIT_TOL, "fused logits")
    # the binary32 level: the summation bound over |x| |w| (sign bits cleared)
    absref = oracle.route_gate(want["out"] & 0x7FFF, w & 0x7FFF)
    assert_dot_bound(lgh, ref, absref, w.shape[1], "fused logits (binary32 level)")
    widx, ww = oracle.route_topk(lgh, K, 1, renorm)
    assert np.array_equal(host(idx), widx)
    np.testing.assert_allclose(host(wt), ww, rtol=1e-5, atol=1e-7)
    if ec is not None:
        assert int(local.item()) == oracle.lar_count(widx, K, 1, want["row_cluster"], ec)


# (n, d, P, G, E, K): one row; less than a workgroup; the tiny workload's
# shape; a ragged 16-byte-vector tail; every supported P; E from 1 to 64;
# K from 1 to 16; the router rows at the 64 KiB limit; the Mixtral-8x7B
# shape (4096 rows of 4096, E = 8, K = 2) and more rows than one pass of the
# grid covers (each wave loops)
CASES = [(1, 128, 2, 2, 4, 2), (7, 64, 1, 3, 3, 1), (64, 128, 2, 2, 4, 2),
         (1000, 520, 2, 8, 8, 2), (777, 384, 4, 5, 16, 4), (333, 1024, 1, 8, 32, 8),
         (129, 2048, 4, 3, 16, 16), (500, 512, 2, 4, 64, 6), (300, 256, 2, 256, 1, 1),
         (4096, 4096, 2, 4, 8, 2), (9000, 256, 2, 8, 8, 2),
         # the matrix-core kernel (65..160 experts, d % 128 == 0), with the
         # top-K in its epilogue: the DeepSeek-V2 width, K up to 16, every P,
         # a ragged last tile, one row
         (1000, 512, 2, 8, 160, 6), (777, 384, 4, 5, 150, 8), (513, 1024, 1, 8, 100, 16),
         (2049, 5120, 2, 8, 160, 6), (64, 128, 2, 2, 65, 1), (1, 256, 2, 3, 160, 6)]


@pytest.mark.parametrize("n,d,P,G,E,K", CASES)
def test_srs_route_against_oracle(n, d, P, G, E, K):
    parts, dest, w, ec = _inputs(n, d, P, G, E)
    got, local = _run(parts, dest, G, w, K, ec)
    _check(parts, dest, G, w, K, ec, 1, got, local)


@pytest.mark.parametrize("E,K", [(12, 3), (160, 6)])
def test_srs_route_full_softmax_and_no_count(E, K):
    """renorm = 0 (softmax over all E, read at the picks); no count."""
    n, d, P, G = 700, 640, 2, 4
    parts, dest, w, _ = _inputs(n, d, P, G, E)
    got, local = _run(parts, dest, G, w, K, None, renorm=0)
    _check(parts, dest, G, w, K, None, 0, got, local)


@pytest.mark.parametrize("E,K", [(160, 6), (150, 8)])
def test_srs_route_matrix_core_equals_separate_calls(E, K):
    """The matrix-core path against srs_shuffle_gate + route_topk + lar_count
    on the GPU: the logits are the same kernel's, so the picks match bit for
    bit; the weights too where route_topk has a fixed-shape kernel of the
    same arithmetic (160 experts, K = 6), else within a few ulp."""
    n, d, P, G = 3000, 1024, 2, 8
    parts, dest, w, ec = _inputs(n, d, P, G, E)
    (out, offs, ros, sor, rc, lg, idx, wt), local = _run(parts, dest, G, w, K, ec)
    o2, f2, r2, s2, c2, l2 = tr.srs_shuffle_gate(dev(parts), dev(dest), G, dev(w))
    i2, w2 = tr.route_topk(l2, K, 1, 1)
    loc2 = torch.zeros(1, dtype=torch.int64, device="cuda")
    tr.lar_count(i2, 1, c2, dev(ec), loc2)
    sync()
    assert torch.equal(out, o2) and torch.equal(lg, l2) and torch.equal(idx, i2)
    if (E, K) == (160, 6):
        assert torch.equal(wt, w2)
    else:
        np.testing.assert_allclose(host(wt), host(w2), rtol=1e-6, atol=1e-8)
    assert int(local.item()) == int(loc2.item())


@pytest.mark.parametrize("E", [8, 160])
def test_srs_route_without_logits(E):
    """Leaving the logits out changes nothing else: the same picks, weights
    and count as the call that writes them (itself checked against the
    oracle)."""
    n, d, P, G, K = 640, 1024, 2, 4, 2
    parts, dest, w, ec = _inputs(n, d, P, G, E)
    got, local = _run(parts, dest, G, w, K, ec)
    _check(parts, dest, G, w, K, ec, 1, got, local)
    got2, local2 = _run(parts, dest, G, w, K, ec, with_logits=False)
    assert got2[5] is None
    assert torch.equal(got[0], got2[0]) and torch.equal(got[6], got2[6])
    assert torch.equal(got[7], got2[7]) and int(local.item()) == int(local2.item())


def test_srs_route_pure_reduce_without_dest():
    """One cluster, no sort: offsets {0, n} and identity maps written by the
    kernel (the buffers start out holding other values); every row's cluster
    is 0 for the count."""
    n, d, P, E, K = 333, 256, 2, 8, 2
    parts = _bf16((P, n, d), 3 + n)
    w = _bf16((E, d), d, 1 / np.sqrt(d))
    ec = np.array([0, 1, 0, 2, 0, 1, 1, 0], dtype=np.uint8)
    fill = lambda k, dt: torch.full((k,), 7, dtype=dt, device="cuda")
    got, local = _run(parts, None, 1, w, K, ec, offsets=fill(2, torch.int32),
                      row_of_src=fill(n, torch.int32), src_of_row=fill(n, torch.int32),
                      row_cluster=fill(n, torch.uint8))
    _check(parts, None, 1, w, K, ec, 1, got, local)


@pytest.mark.parametrize("E", [16, 160])
def test_srs_route_ties_go_to_the_lower_expert(E):
    """Equal router rows give bit-equal logits: the lower index ranks first.
    All-zero rows give +0 logits for every expert (from -0.0 partials too),
    so the picks are experts 0..K-1 with equal weights."""
    n, d, P, G, K = 256, 512, 2, 4, 4
    parts, dest, w, ec = _inputs(n, d, P, G, E)
    w[9] = w[2]
    w[14] = w[2]
    w[5] = w[11]
    parts[:, :40] = 0
    parts[0, 40:60] = 0x8000
    parts[1, 40:60] = 0x8000
    got, local = _run(parts, dest, G, w, K, ec)
    _check(parts, dest, G, w, K, ec, 1, got, local)
    rows = host(got[2])[:60]
    idx, wt = host(got[6])[rows], host(got[7])[rows]
    assert np.all(host(got[5])[rows] == 0)
    assert np.array_equal(idx, np.tile(np.arange(K), (60, 1)))
    np.testing.assert_allclose(wt, 1.0 / K, rtol=1e-6)


def test_srs_route_empty():
    parts = torch.empty((2, 0, 128), dtype=torch.bfloat16, device="cuda")
    dest = torch.empty((0,), dtype=torch.uint8, device="cuda")
    w = dev(_bf16((8, 128), 0))
    r = tr.srs_shuffle_route(parts, dest, 4, w, 2)
    assert host(r[1]).tolist() == [0] * 5 and r[6].shape == (0, 2)


def test_predict_route_and_dispatch_empty():
    """No tokens: the one-launch calls only clear the cluster offsets (and
    the dispatch the expert offsets) and return empty outputs."""
    parts = torch.empty((2, 0, 128), dtype=torch.bfloat16, device="cuda")
    tok = torch.empty((0,), dtype=torch.int32, device="cuda")
    lut = dev(np.zeros(100, np.uint8))
    w = dev(_bf16((8, 128), 0))
    offs = torch.full((5,), 7, dtype=torch.int32, device="cuda")
    r = tr.srs_predict_route(tok, lut, 4, parts, w, 2, offsets=offs)
    eoff = torch.full((9,), 7, dtype=torch.int32, device="cuda")
    offs2 = torch.full((5,), 7, dtype=torch.int32, device="cuda")
    q = tr.srs_predict_route_dispatch(tok, lut, 4, parts, w, 2, offsets=offs2, expert_offsets=eoff)
    sync()
    assert host(r[1]).tolist() == [0] * 5 and r[7].shape == (0, 2)
    assert host(q[1]).tolist() == [0] * 5 and host(q[9]).tolist() == [0] * 9
    assert q[12].shape == (0, 128) and q[10].numel() == 0


@pytest.mark.parametrize("E,K", [(8, 2), (160, 6)])
def test_srs_route_flags_bad_cluster_and_skips_its_row(E, K):
    """A key past G is flagged; its row gets no outputs and adds nothing to
    the count; every other row is exact."""
    n, d, G = 200, 256, 4
    parts, dest, w, ec = _inputs(n, d, 2, G, E)
    dest[7] = 9
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    idx = torch.full((n, K), -5, dtype=torch.int32, device="cuda")
    (out, offs, ros, sor, rc, lg, idx, wt), local = _run(parts, dest, G, w, K, ec, err=err, idx=idx)
    assert int(err.item()) & tr.EBIT_DEST_RANGE
    r = host(ros)
    assert r[7] == -1 and host(offs)[-1] == n - 1
    keep = np.array([i for i in range(n) if i != 7])
    red = oracle.srs_shuffle(parts, np.zeros(n, dtype=np.int64), 1)["out"]
    assert np.array_equal(host(out)[r[keep]], red[keep])
    lgh = host(lg)[r[keep]]
    assert_rel(lgh, oracle.route_gate(red[keep], w), F32_TOL, "logits of the valid rows")
    widx, _ = oracle.route_topk(lgh, K, 1, 1)
    assert np.array_equal(host(idx)[r[keep]], widx)
    free = sorted(set(range(n)) - set(r[keep].tolist()))
    assert len(free) == 1 and np.all(host(idx)[free[0]] == -5)
    assert int(local.item()) == oracle.lar_count(widx, K, 1, dest[keep].astype(np.int64), ec)


@pytest.mark.parametrize("E,K", [(8, 2), (160, 6)])
def test_srs_route_count_accumulates(E, K):
    """The count adds to what the counter holds."""
    n, d, P, G = 500, 256, 2, 4
    parts, dest, w, ec = _inputs(n, d, P, G, E)
    local = torch.full((1,), 1000, dtype=torch.int64, device="cuda")
    r = tr.srs_shuffle_route(dev(parts), dev(dest), G, dev(w), K, expert_cluster=dev(ec), local=local)
    sync()
    want = oracle.srs_shuffle(parts, dest.astype(np.int64), G)
    widx, _ = oracle.route_topk(host(r[5]), K, 1, 1)
    assert int(local.item()) == 1000 + oracle.lar_count(widx, K, 1, want["row_cluster"], ec)


@pytest.mark.filterwarnings("ignore:overflow encountered")   # the oracle's binary32 sums
@pytest.mark.parametrize("kind", ["any_bits", "subnormal_sums"])
def test_srs_route_rows_bit_exact_on_special_values(kind):
    """The reduced rows keep the oracle's bytes on every bf16 pattern: NaN
    (to the canonical 0x7FC0), infinities, overflow to infinity, and sums
    that land among the subnormals (rounded to nearest even there). The
    router results of such rows are outside the contract (NaN logits); only
    the shuffle outputs are compared."""
    n, d, P, G, E, K = 300, 264, 2, 4, 8, 2
    rng = np.random.default_rng(17)
    if kind == "any_bits":
        parts = rng.integers(0, 1 << 16, (P, n, d), dtype=np.int64).astype(np.uint16)
    else:
        sign = rng.integers(0, 2, (P, n, d), dtype=np.int64) << 15
        expo = rng.integers(0, 2, (P, n, d), dtype=np.int64) << 7
        mant = rng.integers(0, 128, (P, n, d), dtype=np.int64)
        parts = (sign | expo | mant).astype(np.uint16)
    dest = rng.integers(0, G, n, dtype=np.int64).astype(np.uint8)
    w = _bf16((E, d), 5, 1 / np.sqrt(d))
    (out, offs, ros, sor, rc, *_), _ = _run(parts, dest, G, w, K, None)
    want = oracle.srs_shuffle(parts, dest.astype(np.int64), G)
    assert np.array_equal(host(offs), want["offsets"])
    assert np.array_equal(host(ros), want["row_of_src"])
    assert np.array_equal(host(out), want["out"])


@pytest.mark.parametrize("n,d,P,G,E,K", [(1000, 520, 2, 8, 8, 2), (777, 384, 4, 5, 16, 4),
                                         (2049, 5120, 2, 8, 160, 6), (300, 256, 2, 3, 150, 8)])
def test_srs_route_sorted_against_oracle(n, d, P, G, E, K):
    """srs_route_sorted on the oracle's own shuffle order: rows, logits,
    picks, weights and count against the oracle (as srs_shuffle_route's
    are), and the same bytes as srs_shuffle_route, through both kernels."""
    parts, dest, w, ec = _inputs(n, d, P, G, E)
    want = oracle.srs_shuffle(parts, dest.astype(np.int64), G)
    ros_o = torch.from_numpy(want["row_of_src"].astype(np.int32)).cuda()
    loc2 = torch.zeros(1, dtype=torch.int64, device="cuda")
    o2, l2, i2, w2 = tr.srs_route_sorted(dev(parts), ros_o, dev(w), K, 1, dest=dev(dest),
                                         expert_cluster=dev(ec), local=loc2)
    sync()
    maps = tuple(torch.from_numpy(np.asarray(want[k]).astype(dt)).cuda() for k, dt in
                 (("offsets", np.int32), ("row_of_src", np.int32), ("src_of_row", np.int32),
                  ("row_cluster", np.uint8)))
    _check(parts, dest, G, w, K, ec, 1, (o2,) + maps + (l2, i2, w2), loc2)
    (out, _, _, _, _, lg, idx, wt), local = _run(parts, dest, G, w, K, ec)
    for a, b in ((out, o2), (lg, l2), (idx, i2), (wt, w2)):
        assert torch.equal(a, b)
    assert int(local.item()) == int(loc2.item())


@pytest.mark.parametrize("n,d,G,E,K,fallback", [(4096, 1024, 4, 8, 2, False),
                                                (5000, 512, 8, 160, 6, True)])
def test_predict_sort_then_route_against_oracle(n, d, G, E, K, fallback):
    """The routed pass's first two calls, route_predict_sort then
    srs_route_sorted, against the oracle's prediction, shuffle, gate, top-K
    and count of the same inputs (one-workgroup and two-launch sorts, the
    lane-per-expert and the matrix-core route kernels)."""
    P, V = 2, 3000
    rng = np.random.default_rng(n + E)
    parts, _, w, ec = _inputs(n, d, P, G, E)
    tok = rng.integers(0, V, n).astype(np.int32)
    lut = rng.integers(0, G, V).astype(np.uint8)
    fb = {}
    conf = prev2 = prev1 = ngram = None
    if fallback:
        conf = rng.integers(0, 256, V).astype(np.uint8)
        prev2 = rng.integers(0, G, n).astype(np.uint8)
        prev1 = rng.integers(0, G, n).astype(np.uint8)
        ngram = rng.integers(0, G, (G, G)).astype(np.uint8)
        fb = dict(conf=dev(conf), prev2=dev(prev2), prev1=dev(prev1), ngram=dev(ngram))
    dest, offs, ros, sor, rc = tr.route_predict_sort(dev(tok), dev(lut), G, **fb)
    local = torch.zeros(1, dtype=torch.int64, device="cuda")
    out, lg, idx, wt = tr.srs_route_sorted(dev(parts), ros, dev(w), K, 1, dest=dest,
                                           expert_cluster=dev(ec), local=local)
    sync()
    want_dest = oracle.route_predict(tok, lut, conf, prev2, prev1, ngram, 128, G=G)
    assert np.array_equal(host(dest), want_dest)
    _check(parts, want_dest.astype(np.uint8), G, w, K, ec, 1,
           (out, offs, ros, sor, rc, lg, idx, wt), local)


def _predict_route_inputs(n, G, V, seed, fallback):
    rng = np.random.default_rng(seed)
    a = dict(tok=rng.integers(0, V, n).astype(np.int32), lut=rng.integers(0, G, V).astype(np.uint8))
    if fallback:
        a.update(conf=rng.integers(0, 256, V).astype(np.uint8),
                 prev2=rng.integers(0, G, n).astype(np.uint8),
                 prev1=rng.integers(0, G, n).astype(np.uint8),
                 ngram=rng.integers(0, G, (G, G)).astype(np.uint8))
    return a


def _two_calls(a, G, parts, w, K, ec, renorm=1):
    fb = {k: dev(a[k]) for k in ("conf", "prev2", "prev1", "ngram") if k in a}
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    dest, offs, ros, sor, rc = tr.route_predict_sort(dev(a["tok"]), dev(a["lut"]), G, err=err, **fb)
    local = torch.zeros(1, dtype=torch.int64, device="cuda")
    out, lg, idx, wt = tr.srs_route_sorted(dev(parts), ros, dev(w), K, renorm, dest=dest,
                                           expert_cluster=None if ec is None else dev(ec),
                                           local=None if ec is None else local)
    return (dest, offs, ros, sor, rc, out, lg, idx, wt), local, err


def _one_call(a, G, parts, w, K, ec, renorm=1):
    fb = {k: dev(a[k]) for k in ("conf", "prev2", "prev1", "ngram") if k in a}
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    local = torch.zeros(1, dtype=torch.int64, device="cuda")
    r = tr.srs_predict_route(dev(a["tok"]), dev(a["lut"]), G, dev(parts), dev(w), K, renorm,
                             expert_cluster=None if ec is None else dev(ec),
                             local=None if ec is None else local, err=err, **fb)
    return r, local, err


# (n, d, P, G, E, K, fallback): one row; a partial workgroup; exactly one and
# one-and-a-bit workgroups; the Mixtral-8x7B shape (4096 rows, the limit);
# 9..16 clusters (two registers of lane counters); one cluster; every P; E
# from 1 to 64; the 2-gram fallback
PRED_CASES = [(1, 128, 2, 2, 4, 2, False), (15, 256, 1, 3, 3, 1, True), (16, 512, 2, 4, 8, 2, False),
              (17, 520, 4, 4, 16, 4, True), (1000, 1024, 2, 9, 32, 8, True),
              (4096, 4096, 2, 4, 8, 2, False), (3000, 256, 2, 16, 64, 6, True),
              (777, 384, 4, 1, 12, 3, False), (2049, 128, 1, 8, 1, 1, True)]


@pytest.mark.parametrize("n,d,P,G,E,K,fallback", PRED_CASES)
def test_predict_route_against_oracle_and_two_calls(n, d, P, G, E, K, fallback):
    """srs_predict_route writes the bytes of route_predict_sort followed by
    srs_route_sorted (every output, the count and the error word), and those
    are the oracle's prediction, shuffle, gate, top-K and count."""
    a = _predict_route_inputs(n, G, 3000, n + G + E, fallback)
    parts, _, w, ec = _inputs(n, d, P, G, E)
    got, local, err = _one_call(a, G, parts, w, K, ec)
    want, local2, err2 = _two_calls(a, G, parts, w, K, ec)
    sync()
    for x, y in zip(got, want):
        assert torch.equal(x, y)
    assert int(local.item()) == int(local2.item())
    assert int(err.item()) == int(err2.item()) == 0
    want_dest = oracle.route_predict(a["tok"], a["lut"], a.get("conf"), a.get("prev2"),
                                     a.get("prev1"), a.get("ngram"), 128, G=G)
    assert np.array_equal(host(got[0]), want_dest)
    dest, offs, ros, sor, rc, out, lg, idx, wt = got
    _check(parts, want_dest.astype(np.uint8), G, w, K, ec, 1,
           (out, offs, ros, sor, rc, lg, idx, wt), local)


@pytest.mark.parametrize("fallback", [False, True])
def test_predict_route_flags_like_two_calls(fallback):
    """Tokens outside the vocabulary, table entries past G and (with the
    fallback) previous clusters past G: the same error bits, maps, rows,
    picks and count as the two calls; renorm = 0 and no count."""
    n, d, P, G, E, K, V = 2500, 512, 2, 4, 16, 4, 3000
    a = _predict_route_inputs(n, G, V, 7, fallback)
    a["tok"][::97] = V + 5
    a["tok"][::131] = -3
    a["lut"][a["tok"][5]] = G + 2
    if fallback:
        a["prev2"][7::211] = G
        a["conf"][:] = np.where(np.arange(V) % 3 == 0, 0, 255).astype(np.uint8)
    parts, _, w, _ = _inputs(n, d, P, G, E)
    got, _, err = _one_call(a, G, parts, w, K, None, renorm=0)
    want, _, err2 = _two_calls(a, G, parts, w, K, None, renorm=0)
    sync()
    e = int(err.item())
    assert e == int(err2.item())
    assert e & tr.EBIT_TOKEN_RANGE and e & tr.EBIT_DEST_RANGE
    dest, offs, ros, sor, rc, out, lg, idx, wt = got
    dest2, offs2, ros2, sor2, rc2, out2, lg2, idx2, wt2 = want
    assert torch.equal(dest, dest2) and torch.equal(offs, offs2) and torch.equal(ros, ros2)
    valid = int(host(offs2)[-1])
    assert valid < n
    assert torch.equal(sor[:valid], sor2[:valid]) and torch.equal(rc[:valid], rc2[:valid])
    for x, y in ((out, out2), (lg, lg2), (idx, idx2), (wt, wt2)):
        assert torch.equal(x[:valid], y[:valid])


@pytest.mark.parametrize("V,shift,fallback", [(3000, 0, True), (3000, 5, False), (60000, 0, True),
                                               (60000, 3, False), (49140, 11, True)])
def test_predict_route_tables_staged_or_not(V, shift, fallback):
    """The token table (and the confidence bytes) are read through LDS when
    they fit (at most 48 KiB from their 16-byte aligned start) and from
    global memory otherwise; tables at any byte alignment. Both ways, every
    output equals the two calls' and the dispatch equals moe_permute's."""
    n, d, P, G, E, K = 2500, 256, 2, 4, 8, 2
    a = _predict_route_inputs(n, G, V, 11 + V + shift, fallback)
    parts, _, w, ec = _inputs(n, d, P, G, E)
    fb = {k: dev(a[k]) for k in ("prev2", "prev1", "ngram") if k in a}

    def shifted(arr):
        buf = torch.zeros(arr.size + 16, dtype=torch.uint8, device="cuda")
        buf[shift:shift + arr.size] = dev(arr)
        return buf[shift:shift + arr.size]
    lut = shifted(a["lut"])
    if fallback:
        fb["conf"] = shifted(a["conf"])
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    local = torch.zeros(1, dtype=torch.int64, device="cuda")
    got = tr.srs_predict_route(dev(a["tok"]), lut, G, dev(parts), dev(w), K, 1,
                               expert_cluster=dev(ec), local=local, err=err, **fb)
    ws = _dispatch_ws(n, G, E)
    err3 = torch.zeros(1, dtype=torch.int32, device="cuda")
    local3 = torch.zeros(1, dtype=torch.int64, device="cuda")
    got3 = tr.srs_predict_route_dispatch(dev(a["tok"]), lut, G, dev(parts), dev(w), K, 1,
                                         expert_cluster=dev(ec), local=local3, write_x=True,
                                         ws=ws, err=err3, **fb)
    want, local2, err2 = _two_calls(a, G, parts, w, K, ec)
    perm = tr.moe_permute(want[7], E, want[5], 1)
    sync()
    assert int(err.item()) == int(err2.item()) == int(err3.item()) == 0
    for x, y, z in zip(got, want, got3[:9]):
        assert torch.equal(x, y) and torch.equal(z, y)
    for x, y in zip(got3[9:], perm):
        assert torch.equal(x, y)
    assert int(local.item()) == int(local2.item()) == int(local3.item())


def _dispatch_call(a, G, parts, w, K, ec, ws, renorm=1, write_x=True):
    fb = {k: dev(a[k]) for k in ("conf", "prev2", "prev1", "ngram") if k in a}
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    local = torch.zeros(1, dtype=torch.int64, device="cuda")
    r = tr.srs_predict_route_dispatch(dev(a["tok"]), dev(a["lut"]), G, dev(parts), dev(w), K,
                                      renorm, expert_cluster=None if ec is None else dev(ec),
                                      local=None if ec is None else local, write_x=write_x,
                                      ws=ws, err=err, **fb)
    return r, local, err


def _dispatch_ws(n, G, E):
    return torch.zeros(tr.srs_predict_route_dispatch_workspace_size(n, G, E), dtype=torch.uint8,
                       device="cuda")


# (n, d, P, G, E, K, fallback): the predict-route cases within 256 (cluster,
# expert) entries: one row (one workgroup, no wait at the barrier); a
# partial workgroup; one and one-and-a-bit workgroups; the Mixtral-8x7B
# shape (4096 rows: 256 workgroups, the most); 256 entries two ways; one
# cluster; every P; E from 1 to 64; K up to 8 (streaming slot stores from 4)
DISP_CASES = [(1, 128, 2, 2, 4, 2, False), (15, 256, 1, 3, 3, 1, True),
              (16, 512, 2, 4, 8, 2, False), (17, 520, 4, 4, 16, 4, True),
              (1000, 1024, 2, 8, 32, 8, True), (4096, 4096, 2, 4, 8, 2, False),
              (3000, 256, 2, 4, 64, 6, True), (777, 384, 4, 1, 12, 3, False),
              (2049, 128, 1, 8, 1, 1, True)]


@pytest.mark.parametrize("n,d,P,G,E,K,fallback", DISP_CASES)
def test_predict_route_dispatch_against_oracle_and_calls(n, d, P, G, E, K, fallback):
    """srs_predict_route_dispatch writes the bytes of srs_predict_route and
    then moe_permute on its rows and picks (every output, the count and the
    error word), and those are the oracle's prediction, shuffle, gate,
    top-K, count and dispatch."""
    a = _predict_route_inputs(n, G, 3000, n + G + E, fallback)
    parts, _, w, ec = _inputs(n, d, P, G, E)
    ws = _dispatch_ws(n, G, E)
    got, local, err = _dispatch_call(a, G, parts, w, K, ec, ws)
    want, local2, err2 = _one_call(a, G, parts, w, K, ec)
    perm = tr.moe_permute(want[7], E, want[5], 1)
    sync()
    for x, y in zip(got[:9], want):
        assert torch.equal(x, y)
    for x, y in zip(got[9:], perm):
        assert torch.equal(x, y)
    assert int(local.item()) == int(local2.item())
    assert int(err.item()) == int(err2.item()) == 0
    assert int(host(ws[:4].view(torch.int32))[0]) % 256 == 0
    want_dest = oracle.route_predict(a["tok"], a["lut"], a.get("conf"), a.get("prev2"),
                                     a.get("prev1"), a.get("ngram"), 128, G=G)
    assert np.array_equal(host(got[0]), want_dest)
    dest, offs, ros, sor, rc, out, lg, idx, wt = got[:9]
    _check(parts, want_dest.astype(np.uint8), G, w, K, ec, 1,
           (out, offs, ros, sor, rc, lg, idx, wt), local)
    x = oracle.srs_shuffle(parts, want_dest.astype(np.int64), G)["out"]
    ref = oracle.moe_permute(oracle.route_topk(host(lg), K, 1, 1)[0], E, 1, src=x[None])
    eoff, sop, pos, disp = got[9:]
    assert np.array_equal(host(eoff), ref["expert_offsets"])
    assert np.array_equal(host(sop), ref["slot_of_pair"])
    assert np.array_equal(host(pos), ref["pair_of_slot"])
    assert np.array_equal(host(disp), ref["disp"])


def test_predict_route_dispatch_calls_in_a_row():
    """One workspace across calls of different grids (256, 7 and 1
    workgroups, then 256 again), with and without the shuffled rows written:
    every call's dispatch equals the separate calls', the error word stays
    clear and the barrier count stays a multiple of 256."""
    G, E, K, d, P = 4, 8, 2, 512, 2
    ws = _dispatch_ws(4096, G, E)
    for i, (n, write_x) in enumerate(((4096, True), (100, False), (9, True), (4096, False))):
        a = _predict_route_inputs(n, G, 3000, 50 + i, i % 2 == 1)
        parts, _, w, ec = _inputs(n, d, P, G, E)
        got, local, err = _dispatch_call(a, G, parts, w, K, ec, ws, write_x=write_x)
        want, local2, err2 = _one_call(a, G, parts, w, K, ec)
        perm = tr.moe_permute(want[7], E, want[5], 1)
        sync()
        assert int(err.item()) == 0 and int(local.item()) == int(local2.item())
        assert (got[5] is None) == (not write_x)
        for j, (x, y) in enumerate(zip(got[:9], want)):
            if x is not None:
                assert torch.equal(x, y), j
        for x, y in zip(got[9:], perm):
            assert torch.equal(x, y)
        assert int(host(ws[:4].view(torch.int32))[0]) == 256 * (i + 1)


def test_predict_route_dispatch_barrier_timeout_flags_sync():
    """The barrier's bounded wait, forced from the host through the
    workspace's bound word. With a bound word of 1 (no poll after a
    workgroup's own arrival), every workgroup but the last to arrive gives
    up, flags SYNC and skips its dispatch, whatever the arrival timing, and
    every kernel still ends. The routing outputs, made before the barrier, are
    whole. The arrival count stays a multiple of 256, and the next call
    with the default bound is whole again."""
    n, d, P, G, E, K = 4096, 512, 2, 4, 8, 2
    a = _predict_route_inputs(n, G, 3000, 5, False)
    parts, _, w, ec = _inputs(n, d, P, G, E)
    ws = _dispatch_ws(n, G, E)
    ws[4:8].view(torch.int32).fill_(1)
    got, local, err = _dispatch_call(a, G, parts, w, K, ec, ws)
    want, local2, err2 = _one_call(a, G, parts, w, K, ec)
    sync()
    assert int(err.item()) == tr.EBIT_SYNC and int(err2.item()) == 0
    assert int(host(ws[:4].view(torch.int32))[0]) % 256 == 0
    for x, y in zip(got[:9], want):
        assert torch.equal(x, y)
    assert int(local.item()) == int(local2.item())
    ws[4:8].view(torch.int32).fill_(0)
    got2, _, err3 = _dispatch_call(a, G, parts, w, K, ec, ws)
    perm = tr.moe_permute(want[7], E, want[5], 1)
    sync()
    assert int(err3.item()) == 0
    for x, y in zip(got2[9:], perm):
        assert torch.equal(x, y)


# (n, d, P, E, K, H, renorm, with_rows): the FoE grouping (64 experts in 4
# groups, K = 8) on its partial count; two and eight groups; one group per
# pick; one row; a ragged last tile; the full softmax (renorm = 0); 160
# experts; the reduced rows written or not
GROUPED_CASES = [(3000, 256, 4, 64, 8, 4, 1, False), (1000, 512, 2, 160, 6, 2, 1, True),
                 (777, 384, 1, 96, 8, 8, 0, True), (65, 128, 4, 64, 4, 4, 0, False),
                 (1, 128, 2, 16, 4, 4, 1, True), (2049, 1024, 4, 64, 8, 4, 1, True),
                 (500, 256, 2, 32, 3, 1, 1, False)]


@pytest.mark.parametrize("n,d,P,E,K,H,renorm,with_rows", GROUPED_CASES)
def test_srs_route_grouped_against_oracle(n, d, P, E, K, H, renorm, with_rows):
    """srs_route_grouped against the oracle's grouped block: the reduced rows
    (when written) bit-exact, the logits against the oracle's gate on them,
    the grouped picks bit-exact and their weights within 1e-5 of the oracle's
    top-K of the kernel's logits, the count exactly lar_count's."""
    from synth import default_expert_cluster, foe_row_cluster
    G = 8
    parts, _, w, _ = _inputs(n, d, P, G, E)
    rc = foe_row_cluster(n, H, G) if H > 1 else np.random.default_rng(n).integers(0, G, n).astype(np.uint8)
    ec = default_expert_cluster(E, G)
    local = torch.zeros(1, dtype=torch.int64, device="cuda")
    out = torch.empty((n, d), dtype=torch.bfloat16, device="cuda") if with_rows else None
    _, lg, idx, wt = tr.srs_route_grouped(dev(parts), dev(w), K, H, renorm, row_cluster=dev(rc),
                                          expert_cluster=dev(ec), local=local, out=out)
    sync()
    red = oracle.srs_shuffle(parts, None, 1)["out"]
    if with_rows:
        assert np.array_equal(host(out), red)
    ref = oracle.route_gate(red, w)
    lgh = host(lg)
    assert_rel(lgh, ref, LOGIT_TOL, "grouped logits")
    assert_dot_bound(lgh, ref, oracle.route_gate(red & 0x7FFF, w & 0x7FFF), d,
                     "grouped logits (binary32 level)")
    widx, ww = oracle.route_topk(lgh, K, H, renorm)
    assert np.array_equal(host(idx), widx)
    np.testing.assert_allclose(host(wt), ww, rtol=1e-5, atol=1e-7)
    assert int(local.item()) == oracle.lar_count(widx, K, H, rc, ec)


def test_srs_route_grouped_equals_separate_calls():
    """On the FoE grouping, against route_topk (H) and lar_count run on the
    kernel's own logits: the picks bit-exact, the weights within a few ulp
    (the same function, another kernel's arithmetic), the count equal."""
    from synth import default_expert_cluster, foe_row_cluster
    n, d, P, E, K, H, G = 3000, 512, 4, 64, 8, 4, 8
    parts, _, w, _ = _inputs(n, d, P, G, E)
    rc = foe_row_cluster(n, H, G)
    ec = default_expert_cluster(E, G)
    local = torch.zeros(1, dtype=torch.int64, device="cuda")
    _, lg, idx, wt = tr.srs_route_grouped(dev(parts), dev(w), K, H, 1, row_cluster=dev(rc),
                                          expert_cluster=dev(ec), local=local)
    i2, w2 = tr.route_topk(lg, K, H, 1)
    loc2 = torch.zeros(1, dtype=torch.int64, device="cuda")
    tr.lar_count(i2, H, dev(rc), dev(ec), loc2)
    sync()
    assert torch.equal(idx, i2)
    np.testing.assert_allclose(host(wt), host(w2), rtol=1e-6, atol=1e-8)
    assert int(local.item()) == int(loc2.item())
