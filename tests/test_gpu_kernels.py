"""GPU parity of every entry point against the oracle, at sizes the oracle
finishes in seconds that span several tiles and a ragged tail, plus edge
cases. Index, permutation, count and bf16-code outputs are bit-exact; the
index stages consume the GPU's own logits / weights. Float outputs use the
tolerances stated in each test."""
import numpy as np
import pytest
import torch

import oracle
import token_routing_speculation_amd as tr
from synth import to_bf16_bits, make_route_inputs
from tests.gpu_helpers import dev, host, assert_rel, assert_bf16, sync

pytestmark = pytest.mark.gpu

LOGIT_TOL = 1e-2      # gate / q_l / estimator: max relative error (row-rms floored)
COMBINE_TOL = 1e-3    # combine, float32 output
WEIGHT_RTOL = 1e-5    # softmax weights (binary32 expf vs float64)


def _bf16(shape, seed, scale=1.0):
    return to_bf16_bits((np.random.default_rng(seed).standard_normal(shape) * scale).astype(np.float32))


# ----------------------------------------------------------------- predict
@pytest.mark.parametrize("n,V,G,fallback", [(1, 5, 2, False), (1000, 512, 2, False),
                                            (4097, 32000, 4, False), (16384, 102400, 8, True),
                                            (777, 300, 256, True)])
def test_predict(n, V, G, fallback):
    rng = np.random.default_rng(n + V)
    tok = rng.integers(0, V, n).astype(np.int32)
    lut = rng.integers(0, G, V, dtype=np.uint8) if G < 256 else rng.integers(0, 256, V, dtype=np.uint8)
    args = {}
    if fallback:
        args = dict(conf=rng.integers(0, 256, V, dtype=np.uint8),
                    prev2=rng.integers(0, G, n, dtype=np.uint8) if G < 256 else rng.integers(0, 256, n, dtype=np.uint8),
                    prev1=rng.integers(0, G, n, dtype=np.uint8) if G < 256 else rng.integers(0, 256, n, dtype=np.uint8),
                    ngram=rng.integers(0, min(G, 256), (G, G), dtype=np.uint8))
    want = oracle.route_predict(tok, lut, args.get("conf"), args.get("prev2"), args.get("prev1"),
                                args.get("ngram"), 128)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    dargs = {k: dev(v.reshape(-1) if k == "ngram" else v) for k, v in args.items()}
    got = tr.route_predict(dev(tok), dev(lut), G, conf_thr=128, err=err, **dargs)
    assert np.array_equal(host(got), want)
    assert int(err.item()) == 0


def test_predict_flags_out_of_vocabulary():
    tok = np.array([0, 5, 2, -1], dtype=np.int32)
    lut = np.array([1, 0, 1], dtype=np.uint8)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    got = host(tr.route_predict(dev(tok), dev(lut), 2, err=err))
    assert got[0] == 1 and got[2] == 1
    assert int(err.item()) & tr.EBIT_TOKEN_RANGE


# ------------------------------------------------------------------- SRS
SRS_CASES = [(1, 8, 1, 1), (7, 136, 2, 2), (1000, 512, 2, 8), (3001, 64, 3, 5), (5000, 256, 4, 1),
             (2049, 40, 5, 256), (4096, 4096, 2, 4), (300, 2048, 1, 7),
             (257, 520, 16, 3), (64, 64, 9, 256),   # the maximum P (16) and a P past the fast paths
             # larger cluster sorts (32 and 33 chunks of 1024 keys)
             (32768, 16, 2, 8), (32769, 16, 2, 8)]


@pytest.mark.parametrize("n,d,P,G", SRS_CASES)
def test_srs_shuffle(n, d, P, G):
    parts = _bf16((P, n, d), n * 31 + d)
    dest = np.random.default_rng(n).integers(0, G, n, dtype=np.uint8) if G <= 255 else \
        np.random.default_rng(n).integers(0, 256, n, dtype=np.uint8)
    want = oracle.srs_shuffle(parts, dest.astype(np.int64), G)
    out, offs, ros, sor, rc = tr.srs_shuffle(dev(parts), dev(dest), G)
    assert np.array_equal(host(offs), want["offsets"])
    assert np.array_equal(host(sor), want["src_of_row"])
    assert np.array_equal(host(ros), want["row_of_src"])
    assert np.array_equal(host(rc), want["row_cluster"])
    assert np.array_equal(host(out), want["out"])


@pytest.mark.parametrize("n,d,P", [(1, 8, 4), (333, 2048, 4), (64, 128, 2), (300, 136, 3),
                                   (70, 4096, 4)])
def test_srs_pure_reduce_without_dest(n, d, P):
    """One cluster, no sort: the row mover itself writes the offsets {0, n}
    and the identity maps (buffers start out holding other values)."""
    parts = _bf16((P, n, d), 5 + n)
    want = oracle.srs_shuffle(parts, None, 1)
    fill = lambda k, dt: torch.full((k,), 7, dtype=dt, device="cuda")
    out, offs, ros, sor, rc = tr.srs_shuffle(dev(parts), None, 1, offsets=fill(2, torch.int32),
                                             row_of_src=fill(n, torch.int32),
                                             src_of_row=fill(n, torch.int32),
                                             row_cluster=fill(n, torch.uint8))
    assert np.array_equal(host(out), want["out"])
    assert host(offs).tolist() == [0, n]
    assert np.array_equal(host(ros), np.arange(n)) and np.array_equal(host(sor), np.arange(n))
    assert np.array_equal(host(rc), np.zeros(n))
    # without maps only the offsets are written
    offs2 = fill(2, torch.int32)
    tr.srs_shuffle(dev(parts), None, 1, offsets=offs2, maps=False)
    assert host(offs2).tolist() == [0, n]


def test_srs_empty():
    parts = torch.empty((2, 0, 64), dtype=torch.bfloat16, device="cuda")
    dest = torch.empty((0,), dtype=torch.uint8, device="cuda")
    _, offs, *_ = tr.srs_shuffle(parts, dest, 4)
    assert host(offs).tolist() == [0] * 5


def test_srs_signed_zero_and_all_one_cluster():
    parts = np.full((2, 100, 16), 0x8000, dtype=np.uint16)
    dest = np.full(100, 3, dtype=np.uint8)
    want = oracle.srs_shuffle(parts, dest, 4)
    out, offs, *_ = tr.srs_shuffle(dev(parts), dev(dest), 4)
    assert np.array_equal(host(out), want["out"]) and host(offs).tolist() == [0, 0, 0, 0, 100]


def test_srs_flags_bad_cluster_and_stays_in_bounds():
    parts = _bf16((2, 50, 16), 1)
    dest = np.zeros(50, dtype=np.uint8)
    dest[7] = 9
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    _, offs, ros, *_ = tr.srs_shuffle(dev(parts), dev(dest), 4, err=err)
    sync()
    assert int(err.item()) & tr.EBIT_DEST_RANGE
    assert host(ros)[7] == -1 and host(offs)[-1] == 49


# ------------------------------------------------------------------- gate
GATE_CASES = [(1, 8, 1), (17, 64, 4), (100, 136, 8), (1000, 520, 17), (4133, 2048, 64),
              (2000, 2048, 128), (1111, 5120, 160), (300, 1024, 200), (64, 256, 1024),
              (4096, 4096, 8), (257, 72, 160),
              # the matrix-core kernel: its shortest K (two steps), one row, a
              # 33-column tile, and its 128 x 128 tiles with ragged rows and columns
              (77, 128, 96), (1, 384, 40), (513, 256, 33), (8200, 1024, 520),
              # its 64 x 160 variant for 129..160 columns: shortest K and one row,
              # ragged rows and columns, ten steps
              (1, 128, 129), (4133, 2048, 150), (65, 640, 160)]


@pytest.mark.parametrize("n,d,E", GATE_CASES)
def test_gate(n, d, E):
    x = _bf16((n, d), n + d)
    w = _bf16((E, d), E + d, 1 / np.sqrt(d))
    got = host(tr.route_gate(dev(x), dev(w)))
    assert_rel(got, oracle.route_gate(x, w), LOGIT_TOL, "gate")
    # the stated bar is loose; binary32 accumulation of exact products is far tighter
    assert_rel(got, oracle.route_gate(x, w), 1e-4, "gate (binary32 level)")


def test_gate_empty_is_noop():
    x = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    w = dev(_bf16((8, 64), 0))
    assert tr.route_gate(x, w).shape == (0, 8)


# ------------------------------------------------------------------- top-K
TOPK_CASES = [(1, 2, 1, 1), (500, 4, 2, 1), (333, 5, 3, 1), (1000, 8, 2, 1), (257, 16, 4, 2),
              (700, 33, 5, 1), (1000, 64, 8, 4), (1000, 64, 2, 1), (999, 128, 8, 1),
              (2048, 160, 6, 1), (400, 160, 6, 2), (100, 1024, 16, 4), (300, 200, 10, 5),
              (64, 7, 7, 1),
              # compile-time-shaped kernels on ragged token counts, and the
              # general kernel on the same E with other K
              (1, 160, 6, 1), (77, 64, 8, 4), (17, 128, 8, 1), (5, 4, 2, 1), (3, 8, 2, 1),
              (300, 160, 4, 1), (129, 128, 4, 1)]


def _tie_logits(n, E, seed):
    rng = np.random.default_rng(seed)
    v = rng.standard_normal((n, E)).astype(np.float32)
    # planted ties: copies of row values, coarse quantisation, signed zeros
    v[: n // 3] = np.round(v[: n // 3] * 2) / 2
    m = rng.random((n, E)) < 0.05
    v[m] = 0.0
    v[(rng.random((n, E)) < 0.05)] = -0.0
    return v


@pytest.mark.parametrize("n,E,K,H", TOPK_CASES)
@pytest.mark.parametrize("renorm", [1, 0])
def test_topk(n, E, K, H, renorm):
    lg = _tie_logits(n, E, n * E + K)
    idx, w = tr.route_topk(dev(lg), K, H, renorm)
    widx, ww = oracle.route_topk(lg, K, H, renorm)
    assert np.array_equal(host(idx), widx)
    np.testing.assert_allclose(host(w), ww, rtol=WEIGHT_RTOL, atol=1e-7)


# ---------------------------------------------------------- permute / combine
PERM_CASES = [(1, 4, 2, 1, 8), (500, 4, 2, 1, 136), (1000, 8, 2, 1, 512), (3000, 160, 6, 1, 64),
              (2000, 64, 8, 4, 128), (1025, 1024, 16, 1, 8), (4096, 16, 4, 2, 40), (77, 3, 3, 1, 16),
              # few experts, many pairs
              (16384, 8, 2, 1, 16), (20000, 8, 2, 1, 16),
              # the one-launch dispatch (at most 16 experts and 16384 pairs) on
              # both sides of its pair limit, with 9..16 experts (two lane
              # counter registers), one expert, groups, ragged rows, and K = 16
              # (a chunk ranked by several waves)
              (8192, 8, 2, 1, 64), (8193, 8, 2, 1, 64), (1024, 16, 16, 1, 24), (3000, 9, 3, 3, 32),
              (33, 1, 1, 1, 8), (2500, 12, 4, 2, 4096), (700, 8, 2, 1, 5120)]


@pytest.mark.parametrize("n,E,K,H,d", PERM_CASES)
def test_permute_and_combine(n, E, K, H, d):
    rng = np.random.default_rng(n + E)
    lg = rng.standard_normal((n, E)).astype(np.float32)
    idx, w = tr.route_topk(dev(lg), K, H, 1)
    src = _bf16((H, n, d), d + n)
    offs, sop, pos, disp = tr.moe_permute(idx, E, dev(src), H)
    want = oracle.moe_permute(host(idx), E, H, src)
    assert np.array_equal(host(offs), want["expert_offsets"])
    assert np.array_equal(host(sop), want["slot_of_pair"])
    assert np.array_equal(host(pos), want["pair_of_slot"])
    assert np.array_equal(host(disp), want["disp"])
    # combine, identity experts; with and without the SAG unshuffle
    out_row = rng.permutation(n).astype(np.int32)
    ref = oracle.moe_combine(want["disp"], host(w).astype(np.float64), want["slot_of_pair"], out_row)
    o32 = tr.moe_combine(disp, w, sop, dev(out_row), out_dtype=torch.float32)
    assert_rel(host(o32), ref, COMBINE_TOL, "combine f32")
    o16 = tr.moe_combine(disp, w, sop, dev(out_row), out_dtype=torch.bfloat16)
    assert_bf16(host(o16), ref, "combine bf16")
    # renormalised identity experts give back the (summed) input exactly
    o16n = host(tr.moe_combine(disp, w, sop))
    if H == 1:
        assert np.array_equal(o16n, src[0])
    # the gather form of the unshuffle (row t combines token in_row[t]): the
    # scatter form's bytes, both output types
    in_row = np.empty(n, dtype=np.int32)
    in_row[out_row] = np.arange(n, dtype=np.int32)
    g16 = tr.moe_combine(disp, w, sop, in_row=dev(in_row))
    assert np.array_equal(host(g16), host(o16))
    g32 = tr.moe_combine(disp, w, sop, in_row=dev(in_row), out_dtype=torch.float32)
    assert np.array_equal(host(g32), host(o32))


@pytest.mark.parametrize("K,d", [(2, 4096), (6, 5120), (8, 128), (3, 136), (1, 8)])
def test_combine_gather_form(K, d):
    """moe_combine_gather against the oracle's combine (rows placed by the
    inverse map) and against the scatter form's bytes, for the instantiated
    K (2, 6, 8) and the plain loop (3, 1), full and ragged rows."""
    n = 777
    rng = np.random.default_rng(K * 1000 + d)
    y = _bf16((n * K, d), K + d)
    w = rng.random((n, K)).astype(np.float32)
    sop = rng.permutation(n * K).astype(np.int32)
    out_row = rng.permutation(n).astype(np.int32)
    in_row = np.empty(n, dtype=np.int32)
    in_row[out_row] = np.arange(n, dtype=np.int32)
    ref = oracle.moe_combine(y, w.astype(np.float64), sop, out_row)
    g = tr.moe_combine(dev(y), dev(w), dev(sop), in_row=dev(in_row))
    assert_bf16(host(g), ref, "combine gather bf16")
    s = tr.moe_combine(dev(y), dev(w), dev(sop), out_row=dev(out_row))
    assert np.array_equal(host(g), host(s))


def test_combine_gather_flags_bad_row():
    """An in_row entry out of range is flagged and its output row left as it
    was; every other row is combined."""
    n, K, d = 100, 2, 64
    rng = np.random.default_rng(3)
    y = _bf16((n * K, d), 5)
    w = rng.random((n, K)).astype(np.float32)
    sop = rng.permutation(n * K).astype(np.int32)
    in_row = rng.permutation(n).astype(np.int32)
    in_row[17] = n + 4
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = torch.full((n, d), 2.0, dtype=torch.bfloat16, device="cuda")
    tr.moe_combine(dev(y), dev(w), dev(sop), in_row=dev(in_row), out=out, err=err)
    sync()
    assert int(err.item()) & tr.EBIT_INDEX_RANGE
    o = host(out)
    assert np.all(o[17] == 0x4000)                      # bf16 2.0, untouched
    keep = np.array([t for t in range(n) if t != 17])
    full = oracle.moe_combine(y, w.astype(np.float64), sop, None)
    assert_bf16(o[keep], full[in_row[keep]], "combine gather, valid rows")


def test_permute_indices_only_and_empty():
    idx = torch.empty((0, 2), dtype=torch.int32, device="cuda")
    offs, *_ = tr.moe_permute(idx, 5)
    assert host(offs).tolist() == [0] * 6
    idx = dev(np.array([[3, 1], [1, 0], [3, 2]], dtype=np.int32))
    offs, sop, pos, disp = tr.moe_permute(idx, 4)
    assert disp is None
    assert host(offs).tolist() == [0, 1, 3, 4, 6]
    assert host(pos).tolist() == [3, 1, 2, 5, 0, 4]


def test_permute_flags_bad_expert():
    idx = dev(np.array([[0, 1], [7, 2]], dtype=np.int32))
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    src = dev(_bf16((1, 2, 16), 3))
    offs, sop, pos, disp = tr.moe_permute(idx, 4, src, err=err)
    sync()
    assert int(err.item()) & tr.EBIT_EXPERT_RANGE
    assert host(sop)[2] == -1 and host(offs)[-1] == 3


@pytest.mark.parametrize("n", [3000, 20000])
def test_permute_rows_flag_bad_experts(n):
    """Out-of-range expert ids with rows, in the one-launch dispatch (3000
    pairs) and the sort + move (20000): flagged, slot -1, nothing moved for
    them; the rest dispatched as if they were absent."""
    E, d = 8, 64
    rng = np.random.default_rng(n)
    idx = rng.integers(0, E, (n, 1)).astype(np.int32)
    bad = rng.choice(n, 9, replace=False)
    idx[bad[:5], 0] = E + 3
    idx[bad[5:], 0] = -2
    src = _bf16((1, n, d), n)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    offs, sop, pos, disp = tr.moe_permute(dev(idx), E, dev(src), err=err)
    sync()
    assert int(err.item()) & tr.EBIT_EXPERT_RANGE
    good = np.setdiff1d(np.arange(n), bad)
    ref = oracle.moe_permute(idx[good], E, 1, src[:, good])
    s = host(sop)
    assert np.all(s[bad] == -1)
    assert np.array_equal(host(offs), ref["expert_offsets"])
    assert np.array_equal(s[good], ref["slot_of_pair"])
    assert np.array_equal(host(pos)[: len(good)], good[ref["pair_of_slot"]])
    assert np.array_equal(host(disp)[: len(good)], ref["disp"])


# ------------------------------------------------------------ counters
@pytest.mark.parametrize("n,E,K,H,G", [(1, 4, 2, 1, 2), (5000, 8, 2, 1, 4), (3000, 160, 6, 1, 8),
                                       (4000, 64, 8, 4, 8), (1000, 64, 8, 4, 2)])
def test_lar_count(n, E, K, H, G):
    from synth import default_expert_cluster, foe_row_cluster
    rng = np.random.default_rng(n)
    idx, _ = tr.route_topk(dev(rng.standard_normal((n, E)).astype(np.float32)), K, H)
    rc = foe_row_cluster(n, H, G) if H > 1 else rng.integers(0, G, n).astype(np.uint8)
    ec = default_expert_cluster(E, G)
    local = torch.zeros(1, dtype=torch.int64, device="cuda")
    tr.lar_count(idx, H, dev(rc), dev(ec), local)
    tr.lar_count(idx, H, dev(rc), dev(ec), local)   # accumulates
    assert int(local.item()) == 2 * oracle.lar_count(host(idx), K, H, rc, ec)


@pytest.mark.parametrize("n,E,K", [(1, 4, 1), (8192, 128, 8), (1000, 16, 16)])
def test_hit_count(n, E, K):
    rng = np.random.default_rng(n + K)
    a, _ = tr.route_topk(dev(rng.standard_normal((n, E)).astype(np.float32)), K)
    b, _ = tr.route_topk(dev(rng.standard_normal((n, E)).astype(np.float32)), K)
    hits = torch.zeros(1, dtype=torch.int64, device="cuda")
    tr.hit_count(a, b, hits)
    assert int(hits.item()) == oracle.hit_count(host(a), host(b))
    hits.zero_()
    tr.hit_count(a, a, hits)
    assert int(hits.item()) == n * K


def test_hit_count_duplicates_as_sets():
    p = dev(np.array([[1, 1, 2], [5, 6, 7]], dtype=np.int32))
    t = dev(np.array([[1, 3, 4], [7, 6, 5]], dtype=np.int32))
    hits = torch.zeros(1, dtype=torch.int64, device="cuda")
    tr.hit_count(p, t, hits)
    assert int(hits.item()) == 4


@pytest.mark.parametrize("K", [2, 4, 6, 8])
def test_hit_count_duplicates_even_k(K):
    # the vector-load kernels (even K) on rows with repeated and shared ids
    rng = np.random.default_rng(K)
    p = rng.integers(0, 5, (301, K)).astype(np.int32)
    t = rng.integers(0, 5, (301, K)).astype(np.int32)
    hits = torch.zeros(1, dtype=torch.int64, device="cuda")
    tr.hit_count(dev(p), dev(t), hits)
    assert int(hits.item()) == oracle.hit_count(p, t)


# --------------------------------------------------------- q_l, estimator
@pytest.mark.parametrize("n,d,affine", [(1, 8, False), (100, 128, True), (8192, 2048, False),
                                        (33, 8192, True), (257, 520, True)])
def test_qhidden(n, d, affine):
    rng = np.random.default_rng(d + n)
    r = _bf16((n, d), d)
    dv = (rng.standard_normal(d) * np.sqrt(0.1)).astype(np.float32)
    g = rng.standard_normal(d).astype(np.float32) if affine else None
    b = rng.standard_normal(d).astype(np.float32) if affine else None
    q = tr.route_qhidden(dev(r), dev(dv), None if g is None else dev(g), None if b is None else dev(b), 1e-5)
    ref = oracle.route_qhidden(r, dv, g, b, 1e-5)
    assert_rel(oracle.bf16_to_f64(host(q)), ref, LOGIT_TOL, "q_l")


@pytest.mark.parametrize("n,d,hd,E", [(1, 64, 8, 8), (300, 256, 72, 40), (2048, 2048, 512, 128),
                                        (300, 256, 136, 40), (8200, 1024, 520, 150)])
def test_estimator(n, d, hd, E):
    rng = np.random.default_rng(n + hd)
    q = _bf16((n, d), 1)
    w1 = _bf16((hd, d), 2, 1 / np.sqrt(d))
    w2 = _bf16((E, hd), 3, 1 / np.sqrt(hd))
    b1 = (rng.standard_normal(hd) * 0.1).astype(np.float32)
    b2 = (rng.standard_normal(E) * 0.1).astype(np.float32)
    got = host(tr.route_estimator(dev(q), dev(w1), dev(b1), dev(w2), dev(b2)))
    assert_rel(got, oracle.route_estimator(q, w1, b1, w2, b2), LOGIT_TOL, "estimator")


# ------------------------------------------------------------ table builder
@pytest.mark.parametrize("n,E,K,G", [(1, 4, 2, 2), (1345, 8, 2, 4), (4549, 160, 6, 8), (500, 64, 16, 256)])
def test_lut_build(n, E, K, G):
    rng = np.random.default_rng(n)
    V = 5 * n + 7
    ids = rng.choice(V, n, replace=False).astype(np.int32)
    idx, w = tr.route_topk(dev(rng.standard_normal((n, E)).astype(np.float32)), K)
    ec = rng.integers(0, G, E).astype(np.uint8)
    lut0 = rng.integers(0, G, V).astype(np.uint8)
    conf0 = rng.integers(0, 256, V).astype(np.uint8)
    lut, conf = dev(lut0), dev(conf0)
    tr.route_lut_build(dev(ids), idx, w, dev(ec), G, lut, conf)
    wl, wc = lut0.copy(), conf0.copy()
    oracle.route_lut_build(ids, host(idx), host(w), ec, G, wl, wc)
    assert np.array_equal(host(lut), wl)
    assert np.array_equal(host(conf), wc)


# ------------------------------------------------------------ determinism
@pytest.mark.parametrize("E", [160, 8])
def test_run_twice_bitwise(E):
    inp = make_route_inputs(3000, 256, E, 6 if E > 8 else 2, 2, 8, 5000, 77, ngram=True)
    from token_routing_speculation_amd.pipeline import RoutePass
    p = RoutePass(inp, lut=inp["lut"], conf=inp["conf"])
    p.step()
    keys = ("x", "logits", "idx", "weights", "slot_of_pair", "disp", "out")
    first = {k: host(getattr(p, k)).copy() for k in keys if k != "x" or p.writes_x}
    l1 = int(host(p.local)[0])
    p.step()
    for k, v in first.items():
        assert np.array_equal(host(getattr(p, k)), v), k
    assert int(host(p.local)[0]) == 2 * l1


def test_run_twice_bitwise_foe_and_predictor():
    """The FoE pass and the q_l predictor (fused gate with top-K and hit
    count on a gate layer; q_l, the estimator's two matrix-core products and
    top-K on an estimator layer), each run twice: bitwise-equal outputs, and
    the counters add exactly the same amount both times."""
    from synth import get_config
    from synth.gen import make_foe_inputs, make_predictor_layer
    from token_routing_speculation_amd.pipeline import FoEPass, PredictorPass
    inp = make_foe_inputs(3000, 256, 64, 4, 8, 8, 5000, 13)
    f = FoEPass(inp)
    keys = ("logits", "idx", "weights", "slot_of_pair", "disp", "out")
    f.step()
    first = {k: host(getattr(f, k)).copy() for k in keys}
    l1 = int(host(f.local)[0])
    f.step()
    for k, v in first.items():
        assert np.array_equal(host(getattr(f, k)), v), k
    assert int(host(f.local)[0]) == 2 * l1
    cfg = get_config("qwen3")
    for layer in (0, 10):                           # an estimator layer, a gate layer
        lay = make_predictor_layer(cfg, layer, N=1000)
        p = PredictorPass(1000, cfg.d, cfg.E, cfg.K, cfg.hd).load(lay)
        p.truth_step()
        p.hits.zero_()
        p.step(keep_logits=True)
        first = {k: host(getattr(p, k)).copy() for k in ("logits", "pred")}
        h1 = int(host(p.hits)[0])
        p.step(keep_logits=True)
        for k, v in first.items():
            assert np.array_equal(host(getattr(p, k)), v), (layer, k)
        assert int(host(p.hits)[0]) == 2 * h1, layer


# ------------------------------------------------------------ graph replay
@pytest.mark.parametrize("E,d,routed", [(160, 512, True), (64, 512, True), (96, 520, False),
                                        (8, 512, True)])
def test_graph_replay_matches_eager(E, d, routed):
    """The benchmark replays the pass as a captured graph: every replay, with
    eager work and synchronisations in between, must equal the eager pass
    (the shuffle, router, top-K and count in one kernel: the matrix-core one
    at 160 columns, the lane-per-expert one at 64 and 8, there with the
    prediction and order inside it and the dispatch in one launch; separate
    calls where neither takes the shape)."""
    from token_routing_speculation_amd.pipeline import RoutePass, capture_graph
    inp = make_route_inputs(2000, d, E, 6, 2, 8, 5000, 91, ngram=True)
    p = RoutePass(inp, lut=inp["lut"], conf=inp["conf"])
    assert p.routed == routed
    keys = ("dest", "x", "row_of_src", "logits", "idx", "weights", "slot_of_pair", "disp", "out")
    # (with the dispatch in the route kernel, x is not written)
    keys = tuple(k for k in keys if k != "x" or p.writes_x)
    p.step()
    sync()
    eager = {k: host(getattr(p, k)).copy() for k in keys}
    g = capture_graph(p.step)
    for rep in range(4):
        for k in keys:                      # scribble over the outputs eagerly
            getattr(p, k).view(torch.uint8).fill_(0xA5)
        sync()
        g.replay()
        sync()
        for k in keys:
            assert np.array_equal(host(getattr(p, k)), eager[k]), (rep, k)


def test_graph_replay_matches_eager_dispatch_in_route():
    """The pass with the dispatch inside the route kernel (its grid barrier
    counting on in the workspace from replay to replay) replayed as a
    captured graph equals the eager pass, replay after replay, and the
    unfused pass."""
    from token_routing_speculation_amd.pipeline import RoutePass, capture_graph
    inp = make_route_inputs(2000, 512, 8, 2, 2, 4, 5000, 93, ngram=True)
    p = RoutePass(inp, lut=inp["lut"], conf=inp["conf"], dispatch_in_route=True)
    assert p.STAGES == ("predict_route_dispatch", "combine") and not p.writes_x
    q = RoutePass(inp, lut=inp["lut"], conf=inp["conf"])
    keys = ("dest", "row_of_src", "logits", "idx", "weights", "expert_offsets", "slot_of_pair",
            "pair_of_slot", "disp", "out")
    p.step()
    q.step()
    sync()
    eager = {k: host(getattr(p, k)).copy() for k in keys}
    for k in keys:
        assert np.array_equal(eager[k], host(getattr(q, k))), k
    g = capture_graph(p.step)
    for rep in range(4):
        for k in keys:
            getattr(p, k).view(torch.uint8).fill_(0xA5)
        sync()
        g.replay()
        sync()
        for k in keys:
            assert np.array_equal(host(getattr(p, k)), eager[k]), (rep, k)
    assert int(p.err.item()) == 0


def test_graph_replay_matches_eager_foe():
    """The FoE pass (the grouped routing in one kernel, the dispatch, the
    combine) replayed as a captured graph equals the eager pass, replay after
    replay."""
    from synth.gen import make_foe_inputs
    from token_routing_speculation_amd.pipeline import FoEPass, capture_graph
    inp = make_foe_inputs(3000, 256, 64, 4, 8, 8, 5000, 17)
    f = FoEPass(inp)
    keys = ("logits", "idx", "weights", "slot_of_pair", "pair_of_slot", "disp", "out")
    f.step()
    sync()
    eager = {k: host(getattr(f, k)).copy() for k in keys}
    l1 = int(host(f.local)[0])
    g = capture_graph(f.step)
    for rep in range(4):
        for k in keys:
            getattr(f, k).view(torch.uint8).fill_(0xA5)
        sync()
        before = int(host(f.local)[0])
        g.replay()
        sync()
        for k in keys:
            assert np.array_equal(host(getattr(f, k)), eager[k]), (rep, k)
        assert int(host(f.local)[0]) - before == l1



def test_graph_replay_matches_eager_predictor():
    """The q_l predictor on an estimator layer (the whole estimator in one
    kernel) and on a gate layer, captured as a graph: every replay's picks
    and logits equal the eager step's, and the hit count grows by the same
    amount each replay (the kernels add to it; nothing clears it)."""
    from synth import get_config
    from synth.gen import make_predictor_layer
    from token_routing_speculation_amd.pipeline import PredictorPass, capture_graph
    cfg = get_config("qwen3")
    for layer in (1, 20):
        lay = make_predictor_layer(cfg, layer, N=777)
        p = PredictorPass(777, cfg.d, cfg.E, cfg.K, cfg.hd).load(lay)
        p.truth_step()
        p.hits.zero_()
        p.step(keep_logits=True)
        sync()
        eager = {k: host(getattr(p, k)).copy() for k in ("logits", "pred")}
        h1 = int(p.hits.item())
        g = capture_graph(lambda: p.step(keep_logits=True))
        for rep in range(3):
            p.logits.fill_(-1.0)
            p.pred.fill_(-1)
            before = int(p.hits.item())
            g.replay()
            sync()
            for k, v in eager.items():
                assert np.array_equal(host(getattr(p, k)), v), (layer, rep, k)
            assert int(p.hits.item()) - before == h1, (layer, rep)
