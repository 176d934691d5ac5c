"""GPU parity on the five model-shaped workloads at full size, through the
same pass objects the benchmark times. Index outputs (predicted clusters,
SRS maps and offsets, top-K, LAR, dispatch maps, hit counts) are checked in
full and bit-exact, the index stages consuming the GPU's logits; bf16 row
data (SRS rows, dispatched rows) bit-exact on sampled rows; float outputs
(logits, q_l, combine) within the stated tolerances on sampled rows, which
the oracle computes one by one from its own reduced activations."""
import numpy as np
import pytest
import torch

import oracle
from oracle.pipeline import build_tables
from synth import make_config_inputs, make_predictor_layer, get_config
from token_routing_speculation_amd import moe_combine
from token_routing_speculation_amd.pipeline import RoutePass, FoEPass, PredictorPass
from tests.gpu_helpers import dev, host, assert_rel, assert_bf16, sync

pytestmark = pytest.mark.gpu

LOGIT_TOL = 1e-2
COMBINE_TOL = 1e-3


def _sample(n, k, seed):
    rng = np.random.default_rng(seed)
    s = rng.choice(n, size=min(k, n), replace=False)
    return np.unique(np.concatenate([s, [0, n - 1]]))


@pytest.mark.parametrize("name", ["tiny", "mixtral", "deepseek"])
def test_route_workload(name):
    cfg = get_config(name)
    inp = make_config_inputs(name)
    lut, conf = build_tables(inp)
    N, d, E, K, G = inp["N"], inp["d"], inp["E"], inp["K"], inp["G"]
    p = RoutePass(inp, lut=lut, conf=conf)
    p.step()
    sync()
    assert int(p.err.item()) == 0
    # a1 predicted clusters
    dest = oracle.route_predict(inp["tok"], lut, conf, inp.get("prev2"), inp.get("prev1"),
                                inp.get("ngram"), cfg.conf_thr, G=G)
    assert np.array_equal(host(p.dest), dest)
    # a2 SRS: maps in full, rows on a sample (the oracle reduces those rows)
    order = np.argsort(dest, kind="stable")
    assert np.array_equal(host(p.src_of_row), order)
    ros = host(p.row_of_src)
    assert np.array_equal(ros[order], np.arange(N))
    assert np.array_equal(host(p.cluster_offsets),
                          np.concatenate([[0], np.cumsum(np.bincount(dest, minlength=G))]))
    assert np.array_equal(host(p.row_cluster), dest[order])
    S = _sample(N, 384, cfg.seed)
    xs = oracle.srs_shuffle(inp["partials"][:, S], None, 1)["out"]
    x_gpu = host(p.x)
    assert np.array_equal(x_gpu[ros[S]], xs)
    # a3 gate on the sampled rows
    lg = host(p.logits)
    assert_rel(lg[ros[S]], oracle.route_gate(xs, inp["w"]), LOGIT_TOL, "gate")
    # a4 top-K on the GPU's logits, in full
    widx, ww = oracle.route_topk(lg, K, 1, 1)
    assert np.array_equal(host(p.idx), widx)
    np.testing.assert_allclose(host(p.weights), ww, rtol=1e-5, atol=1e-7)
    # a5 LAR
    local = oracle.lar_count(widx, K, 1, dest[order], inp["expert_cluster"])
    assert int(p.local.item()) == local
    # a6 dispatch maps in full; rows of the sampled tokens
    perm = oracle.moe_permute(widx, E)
    sop = host(p.slot_of_pair)
    assert np.array_equal(host(p.expert_offsets), perm["expert_offsets"])
    assert np.array_equal(sop, perm["slot_of_pair"])
    assert np.array_equal(host(p.pair_of_slot), perm["pair_of_slot"])
    disp = host(p.disp)
    rows = ros[S]                                     # shuffled rows of the sampled tokens
    for k in range(K):
        assert np.array_equal(disp[sop[rows * K + k]], xs)
    # a7 combine (identity experts) with the unshuffle back to token order
    w_gpu = host(p.weights).astype(np.float64)
    ref = np.einsum("sk,sd->sd", w_gpu[rows], oracle.bf16_to_f64(xs))
    out = host(p.out)
    assert_bf16(out[S], ref, "combine bf16")
    o32 = moe_combine(p.disp, p.weights, p.slot_of_pair, out_row=p.src_of_row,
                      out_dtype=torch.float32)
    assert_rel(host(o32)[S], ref, COMBINE_TOL, "combine f32")


def test_foe_workload():
    inp = make_config_inputs("foe")
    N, d, E, K, H = inp["N"], inp["d"], inp["E"], inp["K"], inp["H"]
    p = FoEPass(inp)
    p.step()
    sync()
    assert int(p.err.item()) == 0
    S = _sample(N, 384, 1004)
    rs = oracle.srs_shuffle(inp["x"][:, S], None, 1)["out"]        # cross-group sum r_full
    assert np.array_equal(host(p.r_full)[S], rs)
    lg = host(p.logits)
    assert_rel(lg[S], oracle.route_gate(rs, inp["w"]), LOGIT_TOL, "gate")
    widx, ww = oracle.route_topk(lg, K, H, 1)
    assert np.array_equal(host(p.idx), widx)
    np.testing.assert_allclose(host(p.weights), ww, rtol=1e-5, atol=1e-7)
    assert int(p.local.item()) == oracle.lar_count(widx, K, H, inp["row_cluster"], inp["expert_cluster"])
    perm = oracle.moe_permute(widx, E, H)
    sop = host(p.slot_of_pair)
    assert np.array_equal(sop, perm["slot_of_pair"])
    assert np.array_equal(host(p.expert_offsets), perm["expert_offsets"])
    disp = host(p.disp)
    kg = K // H
    for k in range(K):
        assert np.array_equal(disp[sop[S * K + k]], inp["x"][k // kg][S])
    # combine: sum over all K slots spans the groups (cross-group sum)
    w_gpu = host(p.weights).astype(np.float64)
    xg = oracle.bf16_to_f64(inp["x"][:, S])                        # [H][s][d]
    ref = sum(w_gpu[S, k][:, None] * xg[k // kg] for k in range(K))
    assert_bf16(host(p.out)[S], ref, "combine bf16")


@pytest.mark.parametrize("layer", [0, 3, 4, 46])
def test_predictor_workload(layer):
    cfg = get_config("qwen3")
    lay = make_predictor_layer(cfg, layer)
    p = PredictorPass(cfg.N, cfg.d, cfg.E, cfg.K, cfg.hd).load(lay)
    p.truth_step()
    S = _sample(cfg.N, 256, layer)
    q_ref = oracle.route_qhidden(lay["r"][S], lay["dvec"], eps=cfg.eps)
    qb = oracle.round_bf16(q_ref)
    if lay["estimator"]:
        ref = oracle.route_estimator(qb, lay["w1"], lay["b1"], lay["w2"], lay["b2"])
    else:
        ref = oracle.route_gate(qb, lay["w_next"])
    # the two-call path materialises q_l; check it and its logits
    p.step(fused=False)
    sync()
    assert_rel(oracle.bf16_to_f64(host(p.q)[S]), q_ref, LOGIT_TOL, "q_l")
    assert_rel(host(p.logits)[S], ref, LOGIT_TOL, "predicted logits (two calls)")
    # the pass as benchmarked (gate layers: route_qgate_topk, q kept on chip)
    p.hits.zero_()
    p.step(keep_logits=True)
    sync()
    lg = host(p.logits)
    assert_rel(lg[S], ref, LOGIT_TOL, "predicted logits")
    tl = host(p.true_logits)
    assert_rel(tl[S], oracle.route_gate(lay["s_next"][S], lay["w_next"]), LOGIT_TOL, "true logits")
    pred, _ = oracle.route_topk(lg, cfg.K, 1, 1)
    truth, _ = oracle.route_topk(tl, cfg.K, 1, 1)
    assert np.array_equal(host(p.pred), pred)
    assert np.array_equal(host(p.truth), truth)
    assert int(p.hits.item()) == oracle.hit_count(pred, truth)
