"""GPU parity on the five model-shaped workloads at full size, through the
same pass objects the benchmark times. Every output is compared in full:
index outputs (predicted clusters, SRS maps and offsets, top-K, LAR,
dispatch maps, hit counts) bit-exact, the index stages consuming the GPU's
logits; bf16 row data (SRS rows, the FoE cross-group sum, dispatched rows)
bit-exact on all rows; float outputs on all rows within the stated
tolerances: logits and q_l at 1e-2, the float32 combine at 1e-3 (both
relative, row-rms floored), the bf16 combine at one bf16 ulp of the
oracle's nearest-even value, with the elements that pass only through the
row floor printed and bounded.

The combine reference is the oracle's ``moe_combine`` applied token block by
token block (the definition is per token) to the oracle's own dispatched
rows and the weights the GPU's top-K wrote (themselves checked against the
oracle's softmax at 1e-5)."""
import numpy as np
import pytest
import torch

import oracle
from oracle.pipeline import build_tables
from synth import make_config_inputs, make_predictor_layer, get_config
from token_routing_speculation_amd import moe_combine
from token_routing_speculation_amd.pipeline import RoutePass, FoEPass, PredictorPass
from tests.gpu_helpers import host, assert_rel, assert_bf16, sync

pytestmark = pytest.mark.gpu

LOGIT_TOL = 1e-2
COMBINE_TOL = 1e-3


def combine_ref(disp, w, slot_of_pair, out_row=None, block=2048):
    """oracle.moe_combine over blocks of tokens: each block's K slots are
    gathered and renumbered, combined, and placed at out_row (SAG)."""
    N, K = w.shape
    out = np.empty((N, disp.shape[1]), dtype=np.float64)
    for a in range(0, N, block):
        b = min(N, a + block)
        rows = disp[slot_of_pair[a * K:b * K]]
        o = oracle.moe_combine(rows, w[a:b], np.arange((b - a) * K))
        if out_row is None:
            out[a:b] = o
        else:
            out[out_row[a:b]] = o
    return out


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
    # a2 SRS: maps and every reduced row
    srs = oracle.srs_shuffle(inp["partials"], dest, G)
    assert np.array_equal(host(p.src_of_row), srs["src_of_row"])
    assert np.array_equal(host(p.row_of_src), srs["row_of_src"])
    assert np.array_equal(host(p.cluster_offsets), srs["offsets"])
    assert np.array_equal(host(p.row_cluster), srs["row_cluster"])
    if p.writes_x:
        # (with the dispatch in the route kernel the shuffled rows are not
        # written: every one of them reaches its K slots, checked below)
        assert np.array_equal(host(p.x), srs["out"])
    x = srs["out"]
    # a3 gate, every row (float64 product of the oracle's rows)
    lg = host(p.logits)
    assert_rel(lg, oracle.route_gate(x, inp["w"]), LOGIT_TOL, "gate")
    # a4 top-K on the GPU's logits
    widx, ww = oracle.route_topk(lg, K, 1, 1)
    assert np.array_equal(host(p.idx), widx)
    np.testing.assert_allclose(host(p.weights), ww, rtol=1e-5, atol=1e-7)
    # a5 LAR
    assert int(p.local.item()) == oracle.lar_count(widx, K, 1, srs["row_cluster"],
                                                   inp["expert_cluster"])
    # a6 dispatch maps and every dispatched row
    perm = oracle.moe_permute(widx, E, 1, src=x[None])
    assert np.array_equal(host(p.expert_offsets), perm["expert_offsets"])
    assert np.array_equal(host(p.slot_of_pair), perm["slot_of_pair"])
    assert np.array_equal(host(p.pair_of_slot), perm["pair_of_slot"])
    assert np.array_equal(host(p.disp), perm["disp"])
    # a7 combine (identity experts) with the unshuffle back to token order
    w_gpu = host(p.weights).astype(np.float64)
    ref = combine_ref(perm["disp"], w_gpu, perm["slot_of_pair"], srs["src_of_row"])
    assert_bf16(host(p.out), ref, "combine bf16", max_floor_frac=1e-5)
    o32 = moe_combine(p.disp, p.weights, p.slot_of_pair, out_row=p.src_of_row,
                      out_dtype=torch.float32)
    assert_rel(host(o32), ref, COMBINE_TOL, "combine f32", max_floor_frac=1e-5)


def test_foe_workload():
    inp = make_config_inputs("foe")
    N, d, E, K, H = inp["N"], inp["d"], inp["E"], inp["K"], inp["H"]
    p = FoEPass(inp)
    p.step()
    sync()
    assert int(p.err.item()) == 0
    # the pass's router reads the cross-group sum r_full on chip (it is not
    # written: test_gpu_srs_route checks those rows where they are written)
    rs = oracle.srs_shuffle(inp["x"], None, 1)["out"]
    lg = host(p.logits)
    assert_rel(lg, oracle.route_gate(rs, inp["w"]), LOGIT_TOL, "gate")
    widx, ww = oracle.route_topk(lg, K, H, 1)
    assert np.array_equal(host(p.idx), widx)
    np.testing.assert_allclose(host(p.weights), ww, rtol=1e-5, atol=1e-7)
    assert int(p.local.item()) == oracle.lar_count(widx, K, H, inp["row_cluster"], inp["expert_cluster"])
    perm = oracle.moe_permute(widx, E, H, src=inp["x"])
    assert np.array_equal(host(p.slot_of_pair), perm["slot_of_pair"])
    assert np.array_equal(host(p.pair_of_slot), perm["pair_of_slot"])
    assert np.array_equal(host(p.expert_offsets), perm["expert_offsets"])
    assert np.array_equal(host(p.disp), perm["disp"])
    # combine: the sum over all K slots spans the groups (cross-group sum); it
    # cancels where the group activations nearly sum to zero, so more
    # elements fall under the row floor than in the plain layout
    w_gpu = host(p.weights).astype(np.float64)
    ref = combine_ref(perm["disp"], w_gpu, perm["slot_of_pair"])
    assert_bf16(host(p.out), ref, "combine bf16", max_floor_frac=1e-3)


@pytest.mark.parametrize("layer", [0, 3, 4, 46])
def test_predictor_workload(layer):
    cfg = get_config("qwen3")
    lay = make_predictor_layer(cfg, layer)
    p = PredictorPass(cfg.N, cfg.d, cfg.E, cfg.K, cfg.hd).load(lay)
    p.truth_step()
    q_ref = oracle.route_qhidden(lay["r"], lay["dvec"], eps=cfg.eps)
    # the two-call path materialises q_l; check it and its logits, every row
    p.step(fused=False)
    sync()
    qg = host(p.q)
    assert_rel(oracle.bf16_to_f64(qg), q_ref, LOGIT_TOL, "q_l")
    qb = oracle.round_bf16(q_ref)
    if lay["estimator"]:
        ref = oracle.route_estimator(qb, lay["w1"], lay["b1"], lay["w2"], lay["b2"])
    else:
        ref = oracle.route_gate(qb, lay["w_next"])
    assert_rel(host(p.logits), ref, LOGIT_TOL, "predicted logits (two calls)")
    # the pass as benchmarked (gate layers: route_qgate_topk, q kept on chip)
    p.hits.zero_()
    p.step(keep_logits=True)
    sync()
    lg = host(p.logits)
    assert_rel(lg, ref, LOGIT_TOL, "predicted logits")
    tl = host(p.true_logits)
    assert_rel(tl, oracle.route_gate(lay["s_next"], lay["w_next"]), LOGIT_TOL, "true logits")
    pred, _ = oracle.route_topk(lg, cfg.K, 1, 1)
    truth, _ = oracle.route_topk(tl, cfg.K, 1, 1)
    assert np.array_equal(host(p.pred), pred)
    assert np.array_equal(host(p.truth), truth)
    assert int(p.hits.item()) == oracle.hit_count(pred, truth)
