"""The fused next gate on q_l ("Speculating Experts Accelerates Inference
for Mixture-of-Experts", item 2.A) against the oracle (float64 q_l and
product, 1e-2 relative with the row floor) and against the two-call path
route_qhidden + route_gate: the bf16 q rows are the same, so the logits may
differ only by the order of the binary32 sums."""

import numpy as np
import pytest
import torch

import token_routing_speculation_amd as tr
import oracle
from oracle.bf16 import round_bf16

from gpu_helpers import dev, host, sync, assert_bf16

pytestmark = pytest.mark.gpu

LOGIT_TOL = 1e-2
TWO_CALL_TOL = 1e-5


def assert_rel(got, ref, tol, what):
    """Elementwise |got - ref| <= tol * max(|ref|, rms of ref): the floor is
    the whole matrix's rms, so rows of one or a few logits (E = 1) are judged
    like the others."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.maximum(np.abs(ref), np.sqrt(np.mean(ref * ref)))
    e = float(np.max(np.abs(got - ref) / den))
    print(f"{what}: max relative error {e:.3e}")
    assert e <= tol, f"{what}: max relative error {e:.3e} > {tol:.1e}"


def _case(n, d, E, affine, seed):
    rng = np.random.default_rng(seed)
    r = round_bf16(rng.standard_normal((n, d)))
    dv = (rng.standard_normal(d) * np.sqrt(0.1)).astype(np.float32)
    g = rng.standard_normal(d).astype(np.float32) if affine else None
    b = rng.standard_normal(d).astype(np.float32) if affine else None
    w = round_bf16(rng.standard_normal((E, d)) / np.sqrt(d))
    return r, dv, g, b, w


@pytest.mark.parametrize("n,d,E,affine", [(1, 2048, 128, False), (8192, 2048, 128, False),
                                          (37, 1024, 8, True), (1000, 4096, 160, True),
                                          (100, 2048, 1, False), (33, 1024, 1024, False),
                                          (77, 2048, 130, True), (16, 4096, 16, False)])
def test_qgate(n, d, E, affine):
    r, dv, g, b, w = _case(n, d, E, affine, n + d + E)
    opt = lambda a: None if a is None else dev(a)
    got = host(tr.route_qgate(dev(r), dev(dv), dev(w), opt(g), opt(b), 1e-5))
    # against the oracle: float64 q_l (not rounded) and a float64 product
    q64 = oracle.route_qhidden(r, dv, g, b, 1e-5)
    want = q64 @ oracle.bf16_to_f64(w).T
    assert_rel(got, want, LOGIT_TOL, "qgate logits")
    # against the two-call path on the same device q
    q = tr.route_qhidden(dev(r), dev(dv), opt(g), opt(b), 1e-5)
    two = host(tr.route_gate(q, dev(w)))
    ref = oracle.bf16_to_f64(host(q)) @ oracle.bf16_to_f64(w).T   # exact products of the bf16 q
    assert_rel(got, ref, TWO_CALL_TOL, "qgate vs the two-call path's bf16 q")
    assert_rel(two, ref, 1e-5, "two-call vs bf16 q")


def test_qgate_top_k_matches_two_call_path():
    """On the Qwen3-shaped next gate the fused and two-call logits pick the
    same top-8 except where two logits sit within float32 rounding."""
    n, d, E, K = 8192, 2048, 128, 8
    r, dv, _, _, w = _case(n, d, E, False, 5)
    a = tr.route_qgate(dev(r), dev(dv), dev(w))
    q = tr.route_qhidden(dev(r), dev(dv))
    bl = tr.route_gate(q, dev(w))
    ia, _ = tr.route_topk(a, K, 1, 1)
    ib, _ = tr.route_topk(bl, K, 1, 1)
    same = (np.sort(host(ia), axis=1) == np.sort(host(ib), axis=1)).all(axis=1)
    assert same.mean() > 0.999


@pytest.mark.parametrize("n,d,E,K,affine", [(1, 2048, 128, 8, False), (8192, 2048, 128, 8, False),
                                            (37, 1024, 8, 2, True), (1000, 4096, 160, 6, True),
                                            (77, 2048, 256, 16, False), (100, 2048, 1, 1, False),
                                            (33, 1024, 200, 5, True), (16, 4096, 64, 8, False)])
def test_qgate_topk_is_route_topk_of_its_logits(n, d, E, K, affine):
    r, dv, g, b, w = _case(n, d, E, affine, n + d + E + K)
    opt = lambda a: None if a is None else dev(a)
    lg = torch.empty((n, E), dtype=torch.float32, device="cuda")
    idx = tr.route_qgate_topk(dev(r), dev(dv), dev(w), K, opt(g), opt(b), 1e-5, logits=lg)
    # the oracle's top-K on the kernel's own logits, bit for bit
    assert np.array_equal(host(idx), oracle.route_topk(host(lg), K, 1, 1)[0])
    want, _ = tr.route_topk(lg, K, 1, 1)
    assert np.array_equal(host(idx), host(want))              # and route_topk's picks
    same = host(tr.route_qgate(dev(r), dev(dv), dev(w), opt(g), opt(b), 1e-5))
    assert np.array_equal(host(lg), same)                     # the same logits as route_qgate
    idx2 = tr.route_qgate_topk(dev(r), dev(dv), dev(w), K, opt(g), opt(b), 1e-5)   # no logits
    assert np.array_equal(host(idx2), host(idx))


@pytest.mark.parametrize("zero_rows", [False, True])
def test_qgate_topk_ties_and_signed_zeros(zero_rows):
    """W rows repeated and zeroed give equal logits and signed zeros; the
    picks are the oracle's on the kernel's logits (lower column on equal
    logits, -0.0 == +0.0) and route_topk's. With ``zero_rows`` only six W
    rows are nonzero (0-4 and 7), so every row's top 8 reaches into the zero logits and
    the tie rule decides most of its picks."""
    n, d, E, K = 64, 1024, 64, 8
    r, dv, _, _, w = _case(n, d, E, False, 9)
    w[20] = 0
    w[21] = 0
    w[22] = 0x8000                         # a row of -0.0
    tied = (10, 40)
    if zero_rows:
        w[5:] = 0
        w[5::2] = 0x8000
        tied = (7,)
    for c in tied:
        w[c] = w[3]
    lg = torch.empty((n, E), dtype=torch.float32, device="cuda")
    idx = tr.route_qgate_topk(dev(r), dev(dv), dev(w), K, logits=lg)
    lgh = host(lg)
    assert all((lgh[:, c] == lgh[:, 3]).all() for c in tied) and (lgh[:, 22] == 0).all()  # ties exist
    picks = host(idx)
    if zero_rows:
        assert (np.take_along_axis(lgh, picks, 1) == 0).sum() >= n   # zero logits are picked
    assert np.array_equal(picks, oracle.route_topk(lgh, K, 1, 1)[0])
    want, _ = tr.route_topk(lg, K, 1, 1)
    assert np.array_equal(picks, host(want))


@pytest.mark.parametrize("n,d,E,K", [(1, 2048, 128, 8), (8192, 2048, 128, 8), (37, 1024, 8, 2),
                                     (1000, 4096, 160, 6), (77, 2048, 256, 16), (100, 2048, 1, 1),
                                     (45, 4096, 64, 3)])
def test_qgate_topk_counts_hits_like_hit_count(n, d, E, K):
    """The fused hit count adds exactly the oracle's |picks & truth| summed
    over rows (integer, bit-exact), computed on the picks the kernel wrote;
    truth rows hold repeats and ids outside 0..E-1 (a repeat counts once, a
    foreign id never), and the counter accumulates."""
    r, dv, _, _, w = _case(n, d, E, False, 3 * n + d + E + K)
    rng = np.random.default_rng(n + K)
    truth = rng.integers(0, E, (n, K)).astype(np.int32)        # repeats allowed
    truth[::7, 0] = E + 3                                       # never a pick
    truth[::5, -1] = -1
    hits = torch.full((1,), 1000, dtype=torch.int64, device="cuda")
    idx = tr.route_qgate_topk(dev(r), dev(dv), dev(w), K, truth=dev(truth), hits=hits)
    picks = host(idx)
    assert int(host(hits)[0]) == 1000 + oracle.hit_count(picks, truth)
    # the picks are those of the call without the count, and hit_count agrees
    assert np.array_equal(host(tr.route_qgate_topk(dev(r), dev(dv), dev(w), K)), picks)
    h2 = torch.zeros(1, dtype=torch.int64, device="cuda")
    tr.hit_count(idx, dev(truth), h2)
    assert int(host(h2)[0]) == oracle.hit_count(picks, truth)


def test_qgate_topk_hits_when_truth_is_the_prediction():
    n, d, E, K = 300, 2048, 128, 8
    r, dv, _, _, w = _case(n, d, E, False, 11)
    idx = tr.route_qgate_topk(dev(r), dev(dv), dev(w), K)
    hits = torch.zeros(1, dtype=torch.int64, device="cuda")
    tr.route_qgate_topk(dev(r), dev(dv), dev(w), K, truth=idx.clone(), hits=hits)
    assert int(host(hits)[0]) == n * K


def _pack_ref(w, d):
    """route_gate_pack's layout written out from its definition: group g of
    16 rows, K step t of 32, lane l holds w[16 g + l % 16][32 t + 8 (l // 16) + e],
    e < 8; rows past E are zeros."""
    E = w.shape[0]
    G = (E + 15) // 16
    wpad = np.zeros((16 * G, d), dtype=np.uint16)
    wpad[:E] = w
    out = np.empty((G, d // 32, 64, 8), dtype=np.uint16)
    for l in range(64):
        rows = 16 * np.arange(G) + (l % 16)
        for t in range(d // 32):
            out[:, t, l, :] = wpad[rows, 32 * t + 8 * (l // 16): 32 * t + 8 * (l // 16) + 8]
    return out.reshape(-1)


@pytest.mark.parametrize("E,d", [(128, 2048), (100, 1024), (1, 32), (256, 4096)])
def test_gate_pack_layout(E, d):
    w = round_bf16(np.random.default_rng(E + d).standard_normal((E, d)))
    wp = tr.route_gate_pack(dev(w))
    assert wp.numel() * 2 == tr.route_gate_packed_size(E, d)
    assert np.array_equal(host(wp), _pack_ref(w, d))


@pytest.mark.parametrize("n,d,E,K,affine", [(1, 2048, 128, 8, False), (8192, 2048, 128, 8, False),
                                            (37, 1024, 8, 2, True), (1000, 4096, 160, 6, True),
                                            (77, 2048, 256, 16, False), (100, 2048, 1, 1, False),
                                            (33, 1024, 200, 5, True), (16, 4096, 64, 8, False)])
def test_qgate_topk_packed_equals_unpacked(n, d, E, K, affine):
    """The packed router gives the unpacked call's logits, picks and hit count
    bit for bit (the same operands in the same order), and its picks are the
    oracle's top-K of those logits."""
    r, dv, g, b, w = _case(n, d, E, affine, 2 * n + d + E + K)
    opt = lambda a: None if a is None else dev(a)
    truth = np.random.default_rng(n + E).integers(0, E, (n, K)).astype(np.int32)
    lg1 = torch.empty((n, E), dtype=torch.float32, device="cuda")
    h1 = torch.zeros(1, dtype=torch.int64, device="cuda")
    i1 = tr.route_qgate_topk(dev(r), dev(dv), dev(w), K, opt(g), opt(b), 1e-5, logits=lg1,
                             truth=dev(truth), hits=h1)
    wp = tr.route_gate_pack(dev(w))
    lg2 = torch.empty((n, E), dtype=torch.float32, device="cuda")
    h2 = torch.zeros(1, dtype=torch.int64, device="cuda")
    i2 = tr.route_qgate_topk_packed(dev(r), dev(dv), wp, E, K, opt(g), opt(b), 1e-5, logits=lg2,
                                    truth=dev(truth), hits=h2)
    assert torch.equal(lg1, lg2) and torch.equal(i1, i2)
    assert int(host(h1)[0]) == int(host(h2)[0])
    assert np.array_equal(host(i2), oracle.route_topk(host(lg2), K, 1, 1)[0])
    assert int(host(h2)[0]) == oracle.hit_count(host(i2), truth)


@pytest.mark.parametrize("n,hd,E,K,with_bias,keep", [(8192, 512, 128, 8, True, True),
                                                     (1, 512, 8, 2, True, False),
                                                     (1000, 1024, 160, 6, False, True),
                                                     (37, 2048, 256, 16, True, True),
                                                     (500, 512, 100, 4, True, False)])
def test_est_out_topk_packed_against_oracle(n, hd, E, K, with_bias, keep):
    """The estimator's output layer with its top-K and hit count in one
    kernel: the logits (when kept) against the oracle's h . w2^T + b2, the
    picks bit-exact against the oracle's top-K of the kernel's own logits
    (kept or recomputed by the two-call form), the hit count exactly
    hit_count's."""
    rng = np.random.default_rng(n + hd + E)
    h = round_bf16(rng.standard_normal((n, hd)) * 0.5)
    w2 = round_bf16(rng.standard_normal((E, hd)) / np.sqrt(hd))
    b2 = (rng.standard_normal(E) * 0.1).astype(np.float32) if with_bias else None
    truth = rng.integers(0, E, (n, K)).astype(np.int32)
    wp = tr.route_gate_pack(dev(w2))
    lg = torch.empty((n, E), dtype=torch.float32, device="cuda") if keep else None
    hits = torch.zeros(1, dtype=torch.int64, device="cuda")
    idx = tr.route_est_out_topk_packed(dev(h), wp, None if b2 is None else dev(b2), E, K, logits=lg,
                                       truth=dev(truth), hits=hits)
    sync()
    ref = oracle.route_gate(h, w2) + (0.0 if b2 is None else b2.astype(np.float64))
    if keep:
        lgh = host(lg)
        assert_rel(lgh, ref, LOGIT_TOL, "estimator output logits")
    else:
        # the same products in the kept form (the logits written, nothing else changes)
        lg2 = torch.empty((n, E), dtype=torch.float32, device="cuda")
        tr.route_est_out_topk_packed(dev(h), wp, None if b2 is None else dev(b2), E, K, logits=lg2)
        sync()
        lgh = host(lg2)
    widx, _ = oracle.route_topk(lgh, K, 1, 1)
    assert np.array_equal(host(idx), widx)
    assert int(hits.item()) == oracle.hit_count(widx, truth)


@pytest.mark.parametrize("n,d,hd,affine", [(1, 2048, 512, False), (8192, 2048, 512, False),
                                           (37, 1024, 8, True), (500, 4096, 200, True),
                                           (77, 2048, 1024, False), (33, 1024, 136, True)])
def test_qest_hidden_packed(n, d, hd, affine):
    """q_l and the estimator's hidden layer in one kernel: h against the
    oracle's GELU(bf16(q_l) W1^T + b1) at the one-ulp bf16 bar (q_l rounded to
    bf16 as route_qhidden stores it), and against route_qhidden +
    route_est_hidden: the same bf16 codes but where the two binary32 sums
    straddle a rounding boundary (one ulp apart, at most 1e-3 of them)."""
    r, dv, g, b, w1 = _case(n, d, hd, affine, 3 * n + d + hd)
    b1 = (np.random.default_rng(hd).standard_normal(hd) * 0.1).astype(np.float32)
    opt = lambda a: None if a is None else dev(a)
    w1p = tr.route_gate_pack(dev(w1))
    h = tr.route_qest_hidden_packed(dev(r), dev(dv), w1p, dev(b1), hd, opt(g), opt(b), 1e-5)
    q = tr.route_qhidden(dev(r), dev(dv), opt(g), opt(b), 1e-5)
    h2 = tr.route_est_hidden(q, dev(w1), dev(b1))
    sync()
    qb = oracle.round_bf16(oracle.route_qhidden(r, dv, g, b, 1e-5))
    qg = host(q)
    # the oracle's hidden layer on the kernel's own bf16 q (q itself is
    # checked against the oracle by the route_qhidden tests)
    ref = oracle.gelu_erf(oracle.bf16_to_f64(qg) @ oracle.bf16_to_f64(w1).T
                          + b1.astype(np.float64)[None, :])
    assert_bf16(host(h), ref, "fused hidden layer")
    a = host(h).view(np.int16).astype(np.int32)
    c = host(h2).view(np.int16).astype(np.int32)
    assert np.abs(a - c).max() <= 1
    assert (a != c).mean() <= 1e-3
    assert (oracle.bf16_to_f64(qg) != oracle.bf16_to_f64(qb)).mean() < 1e-3


@pytest.mark.gpu
@pytest.mark.parametrize("n,d,hd,E,K,affine", [(1, 2048, 512, 128, 8, False),
                                               (8192, 2048, 512, 128, 8, False),
                                               (1000, 2048, 1024, 256, 16, True),
                                               (300, 4096, 512, 200, 8, True),
                                               (77, 1024, 1024, 8, 2, False),
                                               (4097, 1024, 512, 64, 6, True)])
def test_qest_topk_packed(n, d, hd, E, K, affine):
    """The whole estimator predictor in one kernel against
    route_qest_hidden_packed + route_est_out_topk_packed (the same products
    on the same operands in the same order: logits, idx and hits bit for
    bit), and its logits against the oracle's h W2^T + b2 in binary64 on
    that bf16 h, within the bound of a binary32 sum of hd products in any
    order (2 hd 2^-24 sum |h||w|)."""
    r, dv, g, b, w1 = _case(n, d, hd, affine, 5 * n + d + hd + E)
    rng = np.random.default_rng(hd + E)
    b1 = (rng.standard_normal(hd) * 0.1).astype(np.float32)
    w2 = round_bf16(rng.standard_normal((E, hd)) * hd ** -0.5)
    b2 = (rng.standard_normal(E) * 0.1).astype(np.float32)
    truth = rng.integers(0, E, size=(n, K)).astype(np.int32)
    opt = lambda a: None if a is None else dev(a)
    w1p = tr.route_gate_pack(dev(w1))
    w2p = tr.route_gate_pack(dev(w2))
    hits = torch.zeros(1, dtype=torch.int64, device="cuda")
    lg = torch.empty((n, E), dtype=torch.float32, device="cuda")
    idx = tr.route_qest_topk_packed(dev(r), dev(dv), w1p, dev(b1), hd, w2p, dev(b2), E, K,
                                    opt(g), opt(b), 1e-5, logits=lg, truth=dev(truth), hits=hits)
    # the optional outputs left out (no logits, no hit count): the same picks
    idx0 = tr.route_qest_topk_packed(dev(r), dev(dv), w1p, dev(b1), hd, w2p, None if n % 2 else
                                     dev(b2), E, K, opt(g), opt(b), 1e-5)
    h = tr.route_qest_hidden_packed(dev(r), dev(dv), w1p, dev(b1), hd, opt(g), opt(b), 1e-5)
    hits2 = torch.zeros(1, dtype=torch.int64, device="cuda")
    lg2 = torch.empty((n, E), dtype=torch.float32, device="cuda")
    idx2 = tr.route_est_out_topk_packed(h, w2p, dev(b2), E, K, logits=lg2, truth=dev(truth),
                                        hits=hits2)
    sync()
    assert np.array_equal(host(lg).view(np.uint32), host(lg2).view(np.uint32))
    assert np.array_equal(host(idx), host(idx2))
    assert int(hits.item()) == int(hits2.item())
    if n % 2 == 0:
        assert np.array_equal(host(idx0), host(idx))
    else:
        # without b2: the picks of the logits less b2, i.e. of h W2^T alone
        idx0b = tr.route_est_out_topk_packed(h, w2p, None, E, K)
        sync()
        assert np.array_equal(host(idx0), host(idx0b))
    # the picks against the oracle's top-K of the kernel's logits, and the
    # hit count against a count of the picks found among the true ones
    assert np.array_equal(host(idx), oracle.route_topk(host(lg), K, 1, 1)[0])
    assert int(hits.item()) == oracle.hit_count(host(idx), truth)
    hf = oracle.bf16_to_f64(host(h))
    wf = oracle.bf16_to_f64(w2)
    ref = hf @ wf.T + b2.astype(np.float64)[None, :]
    bound = 2.0 * hd * 2.0 ** -24 * (np.abs(hf) @ np.abs(wf).T) + np.abs(ref) * 2.0 ** -23
    assert np.all(np.abs(host(lg).astype(np.float64) - ref) <= bound)
