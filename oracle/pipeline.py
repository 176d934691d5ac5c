"""The oracle's steps composed into whole passes (test infrastructure only).

``route_pass``: predict -> SRS -> gate -> top-K -> LAR -> permute -> combine
with identity experts (the expert output of a slot is its dispatched row).
``foe_pass``: reduce the H group activations -> gate -> grouped top-k/H ->
LAR -> permute from the group activations -> combine (cross-group sum).
``predictor_layer_pass``: q_l -> (next gate | estimator) -> top-K, against the
next layer's true top-K -> hit count.

Where a caller passes ``logits`` the index stages consume those instead of
the oracle's own float64 logits (so a GPU run's logits can be checked
bit-exactly downstream).
"""

from __future__ import annotations

import numpy as np

from .bf16 import round_bf16
from .route import (route_predict, srs_shuffle, route_gate, route_topk, lar_count,
                    moe_permute, moe_combine, route_qhidden, route_estimator,
                    hit_count, route_lut_build)


def build_tables(inp):
    """Fill the token table (and confidence) of a "routing"-mode workload.

    Each occurring id's noiseless activation bf16(base[id]) is routed with the
    gate and top-K; the table builder reduces that routing to a cluster and a
    confidence byte. Returns new (lut, conf) arrays; conf is None when the
    workload has no fallback.
    """
    lut = inp["lut"].copy()
    conf = inp["conf"].copy() if "conf" in inp else None
    if inp.get("lut_mode") != "routing":
        return lut, conf
    logits = route_gate(inp["base_present"], inp["w"])
    idx, w = route_topk(logits, inp["K"], 1, 1)
    route_lut_build(inp["ids_present"], idx, w.astype(np.float32),
                    inp["expert_cluster"], inp["G"], lut, conf)
    return lut, conf


def route_pass(inp, lut, conf=None, logits=None, weights=None):
    G, K, E = inp["G"], inp["K"], inp["E"]
    dest = route_predict(inp["tok"], lut, conf, inp.get("prev2"), inp.get("prev1"),
                         inp.get("ngram"), G=G)
    srs = srs_shuffle(inp["partials"], dest, G)
    own_logits = route_gate(srs["out"], inp["w"])
    lg = own_logits if logits is None else logits
    idx, w = route_topk(lg, K, 1, 1)
    if weights is not None:
        w = weights
    local = lar_count(idx, K, 1, srs["row_cluster"], inp["expert_cluster"])
    perm = moe_permute(idx, E, 1, src=srs["out"][None])
    out = moe_combine(perm["disp"], w, perm["slot_of_pair"], out_row=srs["src_of_row"])
    return dict(dest=dest, srs=srs, logits=own_logits, idx=idx, w=w, local=local,
                perm=perm, out=out)


def foe_pass(inp, logits=None, weights=None):
    H, K, E = inp["H"], inp["K"], inp["E"]
    srs = srs_shuffle(inp["x"], None, 1)
    own_logits = route_gate(srs["out"], inp["w"])
    lg = own_logits if logits is None else logits
    idx, w = route_topk(lg, K, H, 1)
    if weights is not None:
        w = weights
    local = lar_count(idx, K, H, inp["row_cluster"], inp["expert_cluster"])
    perm = moe_permute(idx, E, H, src=inp["x"])
    out = moe_combine(perm["disp"], w, perm["slot_of_pair"])
    return dict(srs=srs, logits=own_logits, idx=idx, w=w, local=local, perm=perm, out=out)


def predictor_layer_pass(layer, pred_logits=None, true_logits=None):
    q = route_qhidden(layer["r"], layer["dvec"], eps=layer["eps"])
    qb = round_bf16(q)
    if layer["estimator"]:
        own = route_estimator(qb, layer["w1"], layer["b1"], layer["w2"], layer["b2"])
    else:
        own = route_gate(qb, layer["w_next"])
    pred, _ = route_topk(own if pred_logits is None else pred_logits, layer["K"], 1, 1)
    true_own = route_gate(layer["s_next"], layer["w_next"])
    truth, _ = route_topk(true_own if true_logits is None else true_logits, layer["K"], 1, 1)
    return dict(q=q, logits=own, pred=pred, true_logits=true_own, truth=truth,
                hits=hit_count(pred, truth))
