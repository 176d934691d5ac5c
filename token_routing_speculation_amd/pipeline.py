"""Whole passes of the routing path, with every buffer allocated up front.

``RoutePass``: predict -> SRS -> gate -> top-K -> LAR -> permute -> combine
(identity experts: the combine reads the dispatched rows themselves), the
s-MoE layer of the "Speculative MoE" notes (section 3.1 and Figure 3's online
path) on one GPU. Where the shapes allow, prediction is folded into the
cluster sort (``predict_sort``) and the SRS, gate, top-K and LAR stages are
one kernel after it (``srs_route``); for small batches all of these are one
kernel (``predict_route``), which can also dispatch the rows to their
expert slots where the (cluster, expert) table is small
(``dispatch_in_route=True``: ``predict_route_dispatch``, the shuffled rows
are then not written).

``FoEPass``: cross-group reduce of the H group activations -> gate ->
grouped top-k/H -> LAR (one kernel, ``route``) -> permute from the group
activations -> combine (cross-group sum), the grouped block of the
"Federation of Experts (FoE)" article.

``ExpertGrouping``: the s-EG expert placement of the "Speculative MoE" notes
(sections 3.2 and 4.2): a token-expert activation profile, then cross-entropy
iterations (sample -> score -> update), all enqueued, and ``grouped_gate`` to
regroup the gate's rows by cluster.

``PredictorPass``: q_l -> next gate (or the estimator on early layers) ->
top-K, and the next layer's true top-K -> hit count ("Speculating Experts
Accelerates Inference for Mixture-of-Experts", items 2.A, 2.C and 4).

Inputs are host numpy arrays from the ``synth`` generator; they are copied to
the device once, in the constructor. ``step()`` enqueues one pass on the
current stream and allocates nothing, so it can be captured once into a HIP
graph (``capture_graph``) and replayed: the same kernels, launched without
per-kernel host overhead.
"""

from __future__ import annotations

import numpy as np
import torch

from . import (route_predict, route_predict_sort, route_lut_build, srs_shuffle,
               srs_shuffle_route, srs_route_sorted, srs_predict_route, srs_route_grouped,
               srs_predict_route_dispatch, srs_predict_route_dispatch_workspace_size,
               route_gate, route_topk, lar_count,
               moe_permute, moe_combine, route_qhidden, route_estimator, hit_count,
               srs_shuffle_workspace_size, moe_permute_workspace_size,
               route_estimator_workspace_size, eg_profile, eg_init, eg_sample, eg_score,
               eg_update, eg_score_workspace_size, route_qgate, route_qgate_topk,
               route_gate_pack, route_qgate_topk_packed, route_est_hidden,
               route_est_out_topk_packed, route_qest_hidden_packed, route_qest_topk_packed)

QGATE_D = (1024, 2048, 4096)  # hidden sizes route_qgate supports


def srs_route_fits(P: int, d: int, E: int, K: int) -> bool:
    """The shapes srs_shuffle_route takes (its UNSUPPORTED rule): one lane per
    expert; the router rows, padded to C * 512 elements (C the smallest of 1,
    2, 4, 8 covering d), within 64 KiB; rows of at most 4096 (2048 with four
    partials); K <= 16."""
    if not (1 <= E <= 64 and 1 <= K <= min(E, 16) and d % 8 == 0 and 8 <= d <= 4096):
        return False
    C = next(c for c in (1, 2, 4, 8) if c * 512 >= d)
    if E * C * 1024 > 65536:
        return False
    return P in (1, 2) or (P == 4 and d <= 2048)


def srs_route_takes(P: int, d: int, E: int, K: int) -> bool:
    """Whether srs_shuffle_route takes the shape at all: the small-set kernel
    (srs_route_fits) or the matrix-core shuffle + router kernel (P in 1, 2,
    4; d % 128 == 0; E <= 160)."""
    if not 1 <= K <= min(E, 16):
        return False
    return srs_route_fits(P, d, E, K) or (P in (1, 2, 4) and d >= 128 and d % 128 == 0
                                          and 1 <= E <= 160)


def predict_route_takes(n: int, P: int, d: int, E: int, K: int, G: int) -> bool:
    """The shapes srs_predict_route takes: at most 4096 tokens and 16
    clusters, on the small-set route kernel (srs_route_fits)."""
    return 0 < n <= 4096 and 1 <= G <= 16 and srs_route_fits(P, d, E, K)


def predict_route_dispatch_takes(n: int, P: int, d: int, E: int, K: int, G: int) -> bool:
    """The shapes srs_predict_route_dispatch takes on the host's checks:
    those of srs_predict_route with at most 256 (cluster, expert) entries
    (the launch also needs its n/16 workgroups resident at once)."""
    return predict_route_takes(n, P, d, E, K, G) and G * E <= 256


def to_device(a: np.ndarray, device="cuda") -> torch.Tensor:
    """numpy -> device tensor; uint16 arrays are bf16 bit patterns."""
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """device bf16 tensor -> host uint16 bit patterns."""
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def capture_graph(step, warmup: int = 2):
    """Capture one call of ``step`` (a pass that allocates nothing and records
    no memset) into a graph; returns the graph, replayed with ``.replay()``."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(warmup):
            step()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    return g


def build_tables_device(inp: dict, device="cuda"):
    """Token -> cluster table (and confidence) from each occurring id's
    noiseless routing: gate + top-K of bf16(base[id]) reduced per cluster by
    route_lut_build ("Speculative MoE" notes, section 4.1)."""
    lut = to_device(inp["lut"], device)
    conf = to_device(inp["conf"], device) if "conf" in inp else None
    if inp.get("lut_mode") != "routing":
        return lut, conf
    base = to_device(inp["base_present"], device)
    w = to_device(inp["w"], device)
    logits = route_gate(base, w)
    idx, wt = route_topk(logits, inp["K"], 1, 1)
    ids = to_device(inp["ids_present"], device)
    ec = to_device(inp["expert_cluster"], device)
    route_lut_build(ids, idx, wt, ec, inp["G"], lut, conf)
    return lut, conf


class RoutePass:
    def __init__(self, inp: dict, lut=None, conf=None, device="cuda", out_dtype=torch.bfloat16,
                 dispatch_in_route=False):
        self.N, self.d, self.E, self.K = inp["N"], inp["d"], inp["E"], inp["K"]
        self.P, self.G = inp["P"], inp["G"]
        N, d, E, K, P, G = self.N, self.d, self.E, self.K, self.P, self.G
        dev = device
        self.tok = to_device(inp["tok"], dev)
        self.partials = to_device(inp["partials"], dev)
        self.w = to_device(inp["w"], dev)
        self.expert_cluster = to_device(inp["expert_cluster"], dev)
        if lut is None:
            lut, conf = build_tables_device(inp, dev)
        self.lut = lut if isinstance(lut, torch.Tensor) else to_device(lut, dev)
        self.conf = None
        self.fallback = conf is not None and "ngram" in inp
        if self.fallback:
            self.conf = conf if isinstance(conf, torch.Tensor) else to_device(conf, dev)
            self.prev2 = to_device(inp["prev2"], dev)
            self.prev1 = to_device(inp["prev1"], dev)
            self.ngram = to_device(inp["ngram"].reshape(-1), dev)
        self.conf_thr = 128
        e = lambda shape, dt: torch.empty(shape, dtype=dt, device=dev)
        self.dest = e((N,), torch.uint8)
        self.x = e((N, d), torch.bfloat16)
        self.cluster_offsets = e((G + 1,), torch.int32)
        self.row_of_src = e((N,), torch.int32)
        self.src_of_row = e((N,), torch.int32)
        self.row_cluster = e((N,), torch.uint8)
        self.ws_srs = e((max(srs_shuffle_workspace_size(N, G), 1),), torch.uint8)
        self.logits = e((N, E), torch.float32)
        self.idx = e((N, K), torch.int32)
        self.weights = e((N, K), torch.float32)
        self.local = torch.zeros((1,), dtype=torch.int64, device=dev)
        self.expert_offsets = e((E + 1,), torch.int32)
        self.slot_of_pair = e((N * K,), torch.int32)
        self.pair_of_slot = e((N * K,), torch.int32)
        self.disp = e((N * K, d), torch.bfloat16)
        self.ws_perm = e((max(moe_permute_workspace_size(N, K, E), 1),), torch.uint8)
        self.out = e((N, d), out_dtype)
        self.err = torch.zeros((1,), dtype=torch.int32, device=dev)
        # the shuffle, router, top-K and count in one kernel after the sort
        # (srs_shuffle_route) where it takes the shape; separate calls
        # otherwise
        self.routed = srs_route_takes(P, d, E, K)
        if self.routed:
            self.STAGES = ("predict_sort", "srs_route", "permute", "combine")
        # small batches: the prediction and the shuffle's order made inside
        # the route kernel (srs_predict_route), one launch for both
        if predict_route_takes(N, P, d, E, K, G):
            self.STAGES = ("predict_route", "permute", "combine")
        # optionally the dispatch in the same kernel too
        # (srs_predict_route_dispatch): the shuffled rows go from registers
        # to their expert slots across a grid barrier, so x is not written.
        # Not the default: on MI355X the barrier's cross-XCD round trips cost
        # about what the rows' write and re-read save at these sizes.
        self.writes_x = True
        if dispatch_in_route and predict_route_dispatch_takes(N, P, d, E, K, G):
            self.STAGES = ("predict_route_dispatch", "combine")
            self.writes_x = False
            self.ws_disp = torch.zeros((srs_predict_route_dispatch_workspace_size(N, G, E),),
                                       dtype=torch.uint8, device=dev)

    def predict(self):
        if self.fallback:
            route_predict(self.tok, self.lut, self.G, self.conf, self.prev2, self.prev1, self.ngram,
                          self.conf_thr, dest=self.dest, err=self.err)
        else:
            route_predict(self.tok, self.lut, self.G, dest=self.dest, err=self.err)

    def srs(self):
        srs_shuffle(self.partials, self.dest, self.G, out=self.x, offsets=self.cluster_offsets,
                    row_of_src=self.row_of_src, src_of_row=self.src_of_row,
                    row_cluster=self.row_cluster, ws=self.ws_srs, err=self.err)

    def gate(self):
        route_gate(self.x, self.w, logits=self.logits)

    def predict_sort(self):
        # the prediction made where the cluster sort reads each key
        fb = dict(conf=self.conf, prev2=self.prev2, prev1=self.prev1, ngram=self.ngram,
                  conf_thr=self.conf_thr) if self.fallback else {}
        route_predict_sort(self.tok, self.lut, self.G, dest=self.dest, offsets=self.cluster_offsets,
                           row_of_src=self.row_of_src, src_of_row=self.src_of_row,
                           row_cluster=self.row_cluster, ws=self.ws_srs, err=self.err, **fb)

    def srs_route(self):
        srs_route_sorted(self.partials, self.row_of_src, self.w, self.K, 1, dest=self.dest,
                         expert_cluster=self.expert_cluster, local=self.local, out=self.x,
                         logits=self.logits, idx=self.idx, weights=self.weights)

    def predict_route(self):
        fb = dict(conf=self.conf, prev2=self.prev2, prev1=self.prev1, ngram=self.ngram,
                  conf_thr=self.conf_thr) if self.fallback else {}
        srs_predict_route(self.tok, self.lut, self.G, self.partials, self.w, self.K, 1,
                          expert_cluster=self.expert_cluster, local=self.local, dest=self.dest,
                          offsets=self.cluster_offsets, row_of_src=self.row_of_src,
                          src_of_row=self.src_of_row, row_cluster=self.row_cluster, out=self.x,
                          logits=self.logits, idx=self.idx, weights=self.weights, err=self.err,
                          **fb)

    def predict_route_dispatch(self):
        fb = dict(conf=self.conf, prev2=self.prev2, prev1=self.prev1, ngram=self.ngram,
                  conf_thr=self.conf_thr) if self.fallback else {}
        srs_predict_route_dispatch(
            self.tok, self.lut, self.G, self.partials, self.w, self.K, 1,
            expert_cluster=self.expert_cluster, local=self.local, dest=self.dest,
            offsets=self.cluster_offsets, row_of_src=self.row_of_src, src_of_row=self.src_of_row,
            row_cluster=self.row_cluster, logits=self.logits, idx=self.idx, weights=self.weights,
            expert_offsets=self.expert_offsets, slot_of_pair=self.slot_of_pair,
            pair_of_slot=self.pair_of_slot, disp=self.disp, ws=self.ws_disp, err=self.err, **fb)

    def topk(self):
        route_topk(self.logits, self.K, 1, 1, idx=self.idx, weights=self.weights)

    def lar(self):
        lar_count(self.idx, 1, self.row_cluster, self.expert_cluster, self.local)

    def permute(self):
        moe_permute(self.idx, self.E, self.x, 1, expert_offsets=self.expert_offsets,
                    slot_of_pair=self.slot_of_pair, pair_of_slot=self.pair_of_slot,
                    disp=self.disp, ws=self.ws_perm, err=self.err)

    def combine(self):
        # the unshuffle in gather form: output row t combines shuffled row
        # row_of_src[t], so the rows are written in order
        moe_combine(self.disp, self.weights, self.slot_of_pair, in_row=self.row_of_src,
                    out=self.out, err=self.err)

    STAGES = ("predict", "srs", "gate", "topk", "lar", "permute", "combine")

    def step(self):
        for s in self.STAGES:
            getattr(self, s)()


class FoEPass:
    def __init__(self, inp: dict, device="cuda", out_dtype=torch.bfloat16):
        self.N, self.d, self.E, self.K, self.H, self.G = (inp["N"], inp["d"], inp["E"], inp["K"],
                                                          inp["H"], inp["G"])
        N, d, E, K, H = self.N, self.d, self.E, self.K, self.H
        dev = device
        self.xg = to_device(inp["x"], dev)
        self.w = to_device(inp["w"], dev)
        self.expert_cluster = to_device(inp["expert_cluster"], dev)
        self.row_cluster = to_device(inp["row_cluster"], dev)
        e = lambda shape, dt: torch.empty(shape, dtype=dt, device=dev)
        self.r_full = e((N, d), torch.bfloat16)
        self.cluster_offsets = e((2,), torch.int32)
        self.ws_srs = e((16,), torch.uint8)
        self.logits = e((N, E), torch.float32)
        self.idx = e((N, K), torch.int32)
        self.weights = e((N, K), torch.float32)
        self.local = torch.zeros((1,), dtype=torch.int64, device=dev)
        self.expert_offsets = e((E + 1,), torch.int32)
        self.slot_of_pair = e((N * K,), torch.int32)
        self.pair_of_slot = e((N * K,), torch.int32)
        self.disp = e((N * K, d), torch.bfloat16)
        self.ws_perm = e((max(moe_permute_workspace_size(N, K, E), 1),), torch.uint8)
        self.out = e((N, d), out_dtype)
        self.err = torch.zeros((1,), dtype=torch.int32, device=dev)

    def route(self):
        # the cross-group reduce, router, grouped top-K and per-group count in
        # one kernel; the reduced rows feed only the router, so they are not
        # written (r_full stays unwritten)
        srs_route_grouped(self.xg, self.w, self.K, self.H, 1, row_cluster=self.row_cluster,
                          expert_cluster=self.expert_cluster, local=self.local,
                          logits=self.logits, idx=self.idx, weights=self.weights)

    def reduce(self):
        srs_shuffle(self.xg, None, 1, out=self.r_full, offsets=self.cluster_offsets, maps=False,
                    ws=self.ws_srs, err=self.err)

    def gate(self):
        route_gate(self.r_full, self.w, logits=self.logits)

    def topk(self):
        route_topk(self.logits, self.K, self.H, 1, idx=self.idx, weights=self.weights)

    def lar(self):
        lar_count(self.idx, self.H, self.row_cluster, self.expert_cluster, self.local)

    def permute(self):
        moe_permute(self.idx, self.E, self.xg, self.H, expert_offsets=self.expert_offsets,
                    slot_of_pair=self.slot_of_pair, pair_of_slot=self.pair_of_slot,
                    disp=self.disp, ws=self.ws_perm, err=self.err)

    def combine(self):
        moe_combine(self.disp, self.weights, self.slot_of_pair, out=self.out, err=self.err)

    # the separate calls (reduce, gate, topk, lar) remain for comparison
    STAGES = ("route", "permute", "combine")

    def step(self):
        for s in self.STAGES:
            getattr(self, s)()


class PredictorPass:
    """One source layer of the q_l predictor; ``load(layer)`` swaps inputs."""

    # estimator layers: q_l, both layers, top-K and the hit count in one
    # kernel where the shape allows (else q_l + hidden, then output + top-K)
    one_kernel_estimator = True

    def __init__(self, N, d, E, K, hd, device="cuda"):
        self.N, self.d, self.E, self.K, self.hd = N, d, E, K, hd
        dev = device
        e = lambda shape, dt: torch.empty(shape, dtype=dt, device=dev)
        self.q = e((N, d), torch.bfloat16)
        self.logits = e((N, E), torch.float32)
        self.true_logits = e((N, E), torch.float32)
        self.pred = e((N, K), torch.int32)
        self.truth = e((N, K), torch.int32)
        self.hits = torch.zeros((1,), dtype=torch.int64, device=dev)
        self.ws = e((max(route_estimator_workspace_size(N, hd), 16),), torch.uint8)
        self.h = e((N, hd), torch.bfloat16)  # the estimator's hidden layer
        self.device = dev
        self.layer = None

    def load(self, layer: dict):
        """Moves the layer's inputs to the device; on gate layers the next
        router is also packed once (route_gate_pack) for the fused kernel,
        like any fixed weight prepared at load time."""
        dev = self.device
        self.layer = {k: (to_device(v, dev) if isinstance(v, np.ndarray) else v)
                      for k, v in layer.items()}
        if not self.layer["estimator"] and self.d in QGATE_D and self.E <= 256:
            self.layer["w_next_packed"] = route_gate_pack(self.layer["w_next"])
        if self.layer["estimator"] and self.hd in (512, 1024, 2048) and self.E <= 256:
            self.layer["w2_packed"] = route_gate_pack(self.layer["w2"])
            if self.d in QGATE_D and self.hd <= 1024:
                self.layer["w1_packed"] = route_gate_pack(self.layer["w1"])
        return self

    def truth_step(self):
        """Layer l+1's own routing (not part of the predictor's pass)."""
        L = self.layer
        route_gate(L["s_next"], L["w_next"], logits=self.true_logits)
        route_topk(self.true_logits, self.K, 1, 1, idx=self.truth, want_weights=False)

    def step(self, fused=True, keep_logits=False):
        """One source layer: on gate layers the next gate on q_l and its top-K
        in one kernel (route_qgate_topk_packed, q and the logits kept on chip; the
        logits are written only if ``keep_logits``) when ``fused`` and the
        shape allows, else route_qhidden + route_gate + route_topk; on
        estimator layers q_l with the hidden layer in one kernel
        (route_qest_hidden_packed, q kept on chip) and the output layer with
        its top-K and hit count in one kernel (route_est_out_topk_packed) when
        ``fused``, else q_l, the estimator and top-K. Then the hit count
        (inside the fused kernels)."""
        L = self.layer
        if not L["estimator"] and fused and "w_next_packed" in L:
            route_qgate_topk_packed(L["r"], L["dvec"], L["w_next_packed"], self.E, self.K,
                                    eps=L["eps"], idx=self.pred,
                                    logits=self.logits if keep_logits else None,
                                    truth=self.truth, hits=self.hits)
            return
        if L["estimator"] and fused and "w2_packed" in L:
            # q_l and the hidden layer in one kernel (q kept on chip) where
            # the shape allows, then the output layer with its top-K and the
            # hit count in one kernel
            if "w1_packed" in L and self.one_kernel_estimator and self.hd in (512, 1024) \
                    and self.hd <= self.d:
                # the whole predictor in one kernel (h kept on chip as well)
                route_qest_topk_packed(L["r"], L["dvec"], L["w1_packed"], L["b1"], self.hd,
                                       L["w2_packed"], L["b2"], self.E, self.K, eps=L["eps"],
                                       idx=self.pred,
                                       logits=self.logits if keep_logits else None,
                                       truth=self.truth, hits=self.hits)
                return
            if "w1_packed" in L:
                route_qest_hidden_packed(L["r"], L["dvec"], L["w1_packed"], L["b1"], self.hd,
                                         eps=L["eps"], h=self.h)
            else:
                route_qhidden(L["r"], L["dvec"], eps=L["eps"], q=self.q)
                route_est_hidden(self.q, L["w1"], L["b1"], h=self.h)
            route_est_out_topk_packed(self.h, L["w2_packed"], L["b2"], self.E, self.K,
                                      logits=self.logits if keep_logits else None,
                                      idx=self.pred, truth=self.truth, hits=self.hits)
            return
        else:
            route_qhidden(L["r"], L["dvec"], eps=L["eps"], q=self.q)
            if L["estimator"]:
                route_estimator(self.q, L["w1"], L["b1"], L["w2"], L["b2"], logits=self.logits,
                                ws=self.ws)
            else:
                route_gate(self.q, L["w_next"], logits=self.logits)
            route_topk(self.logits, self.K, 1, 1, idx=self.pred, want_weights=False)
        hit_count(self.pred, self.truth, self.hits)


class ExpertGrouping:
    """Cross-entropy placement of E experts in G equal clusters from a
    token-expert activation profile. Every step is a library call; ``step``
    and ``solve`` allocate nothing, so an iteration can be captured."""

    def __init__(self, U, E, G, B=256, theta=0.0, rho=0.1, alpha=0.7, seed=0, device="cuda"):
        self.U, self.E, self.G, self.B = U, E, G, B
        self.theta, self.alpha, self.seed = theta, alpha, seed
        self.n_elite = max(1, int(np.ceil(rho * B)))
        z = lambda shape, dt: torch.zeros(shape, dtype=dt, device=device)
        self.counts = z((U, E), torch.int32)
        self.freq = z((U,), torch.int32)
        self.P = z((E, G), torch.float64)
        self.best_J = z((1,), torch.float64)
        self.best_place = z((E,), torch.uint8)
        self.place = z((B, E), torch.uint8)
        self.local = z((B,), torch.int64)
        self.load = z((B, G), torch.int64)
        self.J = z((B,), torch.float64)
        self.ws = z((max(eg_score_workspace_size(U, E, G, B), 16),), torch.uint8)
        self.err = z((1,), torch.int32)
        self.total = 0
        self.tokens = 0

    def profile(self, tok, idx, row_of_id):
        """Adds a routed batch (tok [n] ids, idx [n][K] experts) to the profile."""
        eg_profile(tok, idx, row_of_id, self.counts, self.freq, err=self.err)
        self.total += idx.numel()
        self.tokens += idx.shape[0]

    def reset(self):
        eg_init(self.P, self.best_J)
        self.best_place.zero_()

    def step(self, it):
        eg_sample(self.P, self.B, self.seed, it, place=self.place)
        eg_score(self.counts, self.freq, self.place, self.G, local=self.local, load=self.load,
                 ws=self.ws, err=self.err)
        eg_update(self.local, self.load, self.place, self.total, self.tokens, self.theta,
                  self.n_elite, self.alpha, self.P, self.best_J, self.best_place, J=self.J)

    def solve(self, iters):
        self.reset()
        for it in range(iters):
            self.step(it)
        return self.best_place


def grouped_gate(w, place, G):
    """The gate's rows regrouped by cluster (stable within a cluster): returns
    (w_grouped [E][d], expert_offsets [G+1], new_of_old [E], old_of_new [E]).
    Expert e of the old numbering is row new_of_old[e] of w_grouped, and the
    experts of cluster g are rows expert_offsets[g] .. expert_offsets[g+1]-1."""
    E = w.shape[0]
    keys = place.to(torch.int32).view(E, 1)
    offs, new_of_old, old_of_new, wg = moe_permute(keys, G, w.view(1, E, -1), 1)
    return wg, offs, new_of_old, old_of_new
