#!/usr/bin/env python3
"""Throughput of the MoE routing/dispatch path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input,
already resident in HBM: predict -> SRS (reduce P partials + shuffle into G
cluster ranges) -> gate -> top-K -> LAR -> expert-contiguous dispatch ->
weighted combine with the unshuffle (identity experts). Default workload:
DeepSeek-V2-shaped (N=16384 tokens, d=5120, E=160, K=6, P=2, G=8).

Prints ONE JSON line: routed tokens/s, the per-stage times, the HBM roofline
fraction of the pass and of its dominant kernel, and the CPU oracle timed on
a bounded sample of the same workload on this host.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

HBM_PEAK = 8.0e12            # MI355X HBM3E, bytes/s (AMD spec sheet)
MFMA_BF16_PEAK = 2.5e15      # MI355X dense bf16 matrix throughput, FLOP/s
METRIC = "routed tokens/s (gate->top-K->SRS shuffle->combine) and % of HBM roofline"

ROUTE_WORKLOADS = {"tiny": "tiny", "mixtral": "mixtral-8x7b-shaped", "deepseek": "deepseek-v2-shaped"}


def route_bytes(N, d, E, K, P, G, fallback, routed=False, stages=None):
    """Algorithmic HBM bytes per pass: every call reads its inputs once and
    writes its outputs once (bf16 rows = 2 bytes per element). With the
    shuffle, router, top-K and count in one kernel (srs_shuffle_route) the
    reduced rows are written once and not read back, and neither are the
    logits nor the picks; with the prediction in that kernel too
    (srs_predict_route) the predicted clusters are not read back either; with
    the dispatch in it as well (srs_predict_route_dispatch) the reduced rows
    are not written at all."""
    b = 2
    st = {
        "predict": (9 if fallback else 6) * N,
        "srs": P * N * d * b + N * d * b + 10 * N + 4 * (G + 1),
        "gate": N * d * b + E * d * b + 4 * N * E,
        "topk": 4 * N * E + 8 * N * K,
        "lar": 4 * N * K + N + E,
        "permute": 12 * N * K + 4 * (E + 1) + N * d * b + N * K * d * b,
        "combine": N * K * d * b + 8 * N * K + 4 * N + N * d * b,
    }
    if routed:
        # prediction folded into the cluster sort (its maps: 9 bytes a token
        # and the offsets), then the rows with their router, top-K and count
        rt = {"predict_sort": st["predict"] + 9 * N + 4 * (G + 1),
              "srs_route": (P * N * d * b + N * d * b + E * d * b + 4 * N * E + 8 * N * K
                            + 5 * N + E),
              "permute": st["permute"], "combine": st["combine"]}
        if stages is not None and "predict_route" in stages:
            # both in one kernel: the clusters are not read back (N bytes)
            rt = {"predict_route": rt["predict_sort"] + rt["srs_route"] - N,
                  "permute": rt["permute"], "combine": rt["combine"]}
        if stages is not None and "predict_route_dispatch" in stages:
            # and the dispatch too: the reduced rows go from registers to
            # their K slots (neither written as rows nor read back), the
            # picks are not read back; the two pair maps and the offsets
            rt = {"predict_route_dispatch": (rt["predict_sort"] + rt["srs_route"] - N - N * d * b
                                             + 8 * N * K + 4 * (E + 1) + N * K * d * b),
                  "combine": rt["combine"]}
        return rt
    return st


def foe_bytes(N, d, E, K, H):
    """The FoE pass: the group activations reduced, routed, top-K'd and
    counted in one kernel (the reduced rows are neither written nor read:
    only the router uses them), then the dispatch and the combine."""
    b = 2
    return {
        "route": H * N * d * b + E * d * b + 4 * N * E + 8 * N * K + N * H + E,
        "permute": 12 * N * K + 4 * (E + 1) + H * N * d * b + N * K * d * b,
        "combine": N * K * d * b + 8 * N * K + N * d * b,
    }


ROOT = os.path.dirname(os.path.abspath(__file__))
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_combine_deepseek.json")
TRAFFIC_SOURCES = ("token_routing_speculation_amd/csrc/combine.hip",
                   "token_routing_speculation_amd/csrc/common.hpp")
QGATE_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_qgate_qwen3.json")
QGATE_TRAFFIC_SOURCES = ("token_routing_speculation_amd/csrc/qhidden.hip",
                         "token_routing_speculation_amd/csrc/common.hpp",
                         "token_routing_speculation_amd/csrc/mfma.hpp",
                         "token_routing_speculation_amd/csrc/topk.hpp")


def sources_digest(paths) -> str:
    h = hashlib.sha256()
    for rel in paths:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(workload: str, path=TRAFFIC_FILE, sources=TRAFFIC_SOURCES):
    """HBM bytes per launch of a kernel (the combine by default) from the
    committed counter runs (FETCH_SIZE and WRITE_SIZE, each scaled by what the
    counter reads for a copy of known size), or None when the kernel's sources
    have changed since they were taken or the workload differs."""
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("workload") != workload or rec.get("sha256") != sources_digest(sources):
        return None
    return (rec["fetch_kib"] * 1024 * rec["fetch_scale"] + rec["write_kib"] * 1024 * rec["write_scale"])


def _oracle_passes(name, inp, tables, min_seconds):
    import oracle.pipeline as op
    passes, dt = 0, 0.0
    while dt < min_seconds:
        t0 = time.perf_counter()
        if name == "foe":
            op.foe_pass(inp)
        else:
            op.route_pass(inp, *tables)
        dt += time.perf_counter() - t0
        passes += 1
    return passes, dt


def host_cores() -> int:
    """Cores this process may run on (its CPU affinity set)."""
    return len(os.sched_getaffinity(0))


def blas_threads() -> int:
    from threadpoolctl import threadpool_info
    return int(max([p.get("num_threads", 1) for p in threadpool_info()] or [1]))


def cpu_baseline(name: str, inp: dict, n_sample: int, min_seconds: float = 10.0):
    """The oracle (float64 NumPy, as it stands) on the first n_sample tokens
    of the benchmarked batch itself, full passes repeated until min_seconds of
    host time have been spent. Run with the BLAS pool at its default size (the
    reported value) and again with one thread (threadpoolctl limits the pool
    in-process)."""
    from threadpoolctl import threadpool_limits
    from synth import first_tokens
    import oracle.pipeline as op

    sub = first_tokens(inp, n_sample)
    n = sub["N"]
    tables = None if name == "foe" else op.build_tables(sub)
    passes, dt = _oracle_passes(name, sub, tables, min_seconds)
    threads = blas_threads()
    with threadpool_limits(limits=1):
        passes1, dt1 = _oracle_passes(name, sub, tables, min_seconds / 2)
    return {"value": passes * n / dt, "unit": "tokens/s", "cores": host_cores(),
            "blas_threads": threads, "kind": "oracle",
            "sample": f"{passes} full passes over the first {n} of the {inp['N']} benchmarked "
                      f"tokens of the {name} workload (float64 NumPy; matrix products on "
                      f"{threads} BLAS threads, elementwise steps on one); {dt:.1f} s",
            "value_1_thread": passes1 * n / dt1,
            "sample_1_thread": f"{passes1} passes with the BLAS pool limited to 1 thread; "
                               f"{dt1:.1f} s"}


def pct(xs):
    """10th, 50th and 90th percentile of a list of per-pass times (ms)."""
    q = np.percentile(np.asarray(xs, dtype=np.float64), [10, 50, 90])
    return [round(float(v), 4) for v in q]


def lar_rate(p, pairs):
    """Local activation rate of one pass (the counter accumulates)."""
    p.local.zero_()
    p.step()
    return int(p.local.item()) / pairs


def eg_bench(args):
    """s-EG expert placement ("Speculative MoE" notes, sections 3.2 and 4.2) on
    the DeepSeek-V2-shaped model: profile a held-out routed batch, solve the
    placement by cross-entropy iterations, then route the benchmark batch with
    the default contiguous placement and with the solved one and compare the
    local activation rate and the cluster load balance."""
    import torch
    from synth import make_config_inputs, get_config
    from token_routing_speculation_amd.pipeline import RoutePass, ExpertGrouping

    cfg = get_config(args.config)
    torch.cuda.set_device(0)
    # profile: a held-out batch of the same model, routed by the library
    prof = make_config_inputs(args.config, sample=1)
    pp = RoutePass(prof)
    pp.predict(); pp.srs(); pp.gate(); pp.topk()
    tok_rows = torch.from_numpy(prof["tok"]).cuda()[pp.src_of_row.long()].to(torch.int32)
    ids = np.unique(prof["tok"])
    row_of_id = np.full(cfg.V, -1, np.int32)
    row_of_id[ids] = np.arange(len(ids), dtype=np.int32)
    U = len(ids)
    g = ExpertGrouping(U, cfg.E, cfg.G, B=args.eg_candidates, theta=args.eg_theta, seed=7)
    g.profile(tok_rows, pp.idx, torch.from_numpy(row_of_id).cuda())
    torch.cuda.synchronize()
    del pp
    stream = torch.cuda.current_stream()
    iters = args.eg_iters
    # per-stage times over a few iterations, then the whole solve
    g.reset()
    from token_routing_speculation_amd import eg_sample, eg_score, eg_update
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(5)]
    for it in range(5):
        ev[it][0].record(stream)
        eg_sample(g.P, g.B, g.seed, it, place=g.place)
        ev[it][1].record(stream)
        eg_score(g.counts, g.freq, g.place, g.G, local=g.local, load=g.load, ws=g.ws, err=g.err)
        ev[it][2].record(stream)
        eg_update(g.local, g.load, g.place, g.total, g.tokens, g.theta, g.n_elite, g.alpha,
                  g.P, g.best_J, g.best_place, J=g.J)
        ev[it][3].record(stream)
    torch.cuda.synchronize()
    stage = {n: 1e3 * np.median([ev[i][k].elapsed_time(ev[i][k + 1]) for i in range(1, 5)])
             for k, n in enumerate(("sample", "score", "update"))}
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    best = g.solve(iters)
    e1.record(stream)
    torch.cuda.synchronize()
    solve_ms = e0.elapsed_time(e1)
    place = best.cpu().numpy()

    eval_inp = make_config_inputs(args.config)

    def route_with(expert_cluster):
        inp = dict(eval_inp, expert_cluster=expert_cluster)
        p = RoutePass(inp)
        lar = lar_rate(p, cfg.N * cfg.K)
        offs = p.cluster_offsets.cpu().numpy()
        sizes = np.diff(offs)
        return lar, float(sizes.max() / sizes.mean())

    from synth.gen import default_expert_cluster
    lar0, imb0 = route_with(default_expert_cluster(cfg.E, cfg.G))
    lar1, imb1 = route_with(place.astype(np.uint8))
    # score-stage roofline: the matrix-core product (exact integer counts)
    flops = 2.0 * U * (2 * cfg.E) * g.B * cfg.G
    out = {
        "metric": "s-EG cross-entropy placement: solve time and local activation rate gain",
        "value": iters / (solve_ms * 1e-3), "unit": "solver iterations/s",
        "higher_is_better": True, "n_gpus": 1, "data": "synthetic",
        "config": {"workload": ROUTE_WORKLOADS[args.config], "profile_tokens": cfg.N,
                   "profiled_ids": U, "E": cfg.E, "G": cfg.G, "candidates": g.B,
                   "iterations": iters, "theta": g.theta, "elite": g.n_elite, "alpha": g.alpha},
        "solve_ms": solve_ms, "stage_us": {k: round(v, 2) for k, v in stage.items()},
        "score_gemm_tflops_at_stage_time": flops / (stage["score"] * 1e-6) / 1e12,
        "best_J": float(g.best_J.item()),
        "lar_default_placement": lar0, "lar_eg_placement": lar1,
        "lar_gain": lar1 / lar0 - 1.0,
        "cluster_load_max_over_mean": {"default": imb0, "eg": imb1},
    }
    if not args.no_cpu_baseline:
        from oracle import eg as oeg
        counts = g.counts.cpu().numpy().astype(np.int64)
        freq = g.freq.cpu().numpy().astype(np.int64)
        t0 = time.perf_counter()
        total_its = 2
        oeg.ceo_place(counts, freq, cfg.G, theta=g.theta, B=g.B, iters=total_its, seed=7)
        dt = time.perf_counter() - t0
        out["cpu_baseline"] = {"value": total_its / dt, "unit": "solver iterations/s", "cores": 1,
                               "kind": "oracle",
                               "sample": f"{total_its} oracle iterations (float64 NumPy) on the "
                                         f"same profile; {dt:.1f} s"}
    print(json.dumps(out), flush=True)
    return 0


def predictor_bytes(N, d, E, K, hd, estimator, fused=False):
    """Algorithmic HBM bytes of one source layer's prediction (q_l -> logits ->
    top-K -> hits), each call reading its inputs and writing its outputs once.
    fused: the next gate, its top-K and the hit count as one route_qgate_topk
    (r, d_l, W and the true picks read, the picks written, the counter updated;
    q and the logits never leave the chip)."""
    b = 2
    if fused and not estimator:
        return {"qgate_topk": N * d * b + 4 * d + E * d * b + 4 * N * K + 4 * N * K + 16}
    if fused and hd in (512, 1024) and hd <= d:
        # the whole estimator predictor in one kernel (q, h and the logits
        # never leave the chip)
        return {"qest_topk_hits": N * d * b + 4 * d + hd * d * b + 4 * hd + E * hd * b + 4 * E
                + 8 * N * K + 8}
    if fused:
        # q_l and the hidden layer in one kernel (q never leaves the chip),
        # then the output layer with its top-K and the hit count in one
        # kernel (the logits never leave the chip)
        return {"q_hidden": N * d * b + 4 * d + hd * d * b + 4 * hd + N * hd * b,
                "out_topk_hits": N * hd * b + E * hd * b + 4 * E + 8 * N * K + 8}
    st = {"qhidden": 2 * N * d * b + 4 * d,
          "logits": (N * d * b + hd * d * b + 4 * hd + N * hd * b + E * hd * b + 4 * E + 4 * N * E)
          if estimator else (N * d * b + E * d * b + 4 * N * E),
          "topk": 4 * N * E + 4 * N * K,
          "hits": 8 * N * K + 8}
    return st


def fit_estimator(cfg, l, lay, n_train, ridge, time_oracle=False):
    """Fits layer l's estimator output weights on a held-out batch of the same
    model ("Speculating Experts", item 2.C; ridge regression on the
    estimator's own features) and stores them in ``lay``. Returns timings and
    the hit rate of the gate on q_l for the same layer (the alternative the
    estimator replaces)."""
    import torch
    import token_routing_speculation_amd as tr
    from synth.gen import make_predictor_layer
    from token_routing_speculation_amd.pipeline import to_device

    tr_l = make_predictor_layer(cfg, l, N=n_train, sample=1)
    dev_ = {k: to_device(v) for k, v in tr_l.items() if isinstance(v, np.ndarray)}
    q = tr.route_qhidden(dev_["r"], dev_["dvec"], eps=cfg.eps)
    y = tr.route_gate(dev_["s_next"], dev_["w_next"])
    gram = torch.empty((cfg.hd + 1, cfg.hd + 1), dtype=torch.float64, device="cuda")
    rhs = torch.empty((cfg.hd + 1, cfg.E), dtype=torch.float64, device="cuda")
    ws = torch.empty(tr.est_fit_gram_workspace_size(n_train, cfg.hd, cfg.E), dtype=torch.uint8,
                     device="cuda")
    info = torch.zeros(1, dtype=torch.int32, device="cuda")
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(5)]
    torch.cuda.synchronize()
    ev[0].record()
    h = tr.route_est_hidden(q, dev_["w1"], dev_["b1"])
    ev[1].record()
    tr.est_fit_gram(h, y, gram=gram, rhs=rhs, ws=ws)
    ev[2].record()
    tr.est_fit_solve(gram, rhs, ridge, info=info)
    ev[3].record()
    w2, b2 = tr.est_fit_weights(rhs)
    ev[4].record()
    torch.cuda.synchronize()
    if int(info.item()):
        raise RuntimeError(f"estimator fit of layer {l}: matrix not positive definite")
    lay["w2"] = w2.view(torch.int16).cpu().numpy().view(np.uint16)
    lay["b2"] = b2.cpu().numpy()
    t = [ev[i].elapsed_time(ev[i + 1]) for i in range(4)]
    info = {"train_tokens": n_train, "ridge": ridge, "hidden_ms": t[0], "gram_ms": t[1],
            "solve_ms": t[2], "weights_ms": t[3]}
    if time_oracle:
        # the oracle's float64 fit (Gram, LAPACK solve, rounding) on the same features
        from oracle import estfit as oest
        h_np = h.view(torch.int16).cpu().numpy().view(np.uint16)
        y_np = y.cpu().numpy()
        t0 = time.perf_counter()
        ow2, _, _ = oest.est_fit(h_np, y_np, ridge)
        info["cpu_baseline"] = {"value": (time.perf_counter() - t0) * 1e3, "unit": "ms per fit",
                                "cores": host_cores(), "blas_threads": blas_threads(),
                                "kind": "oracle",
                                "sample": "the same layer's fit, once (float64 NumPy and LAPACK)",
                                "bf16_codes_equal": float((ow2 == lay["w2"]).mean())}
    return info


def predictor_setup(cfg, args):
    """The predictor pass and every source layer's device inputs, with layer
    l+1's true top-K (its own routing) computed once; optionally the
    estimator layers' output weights fitted first."""
    import torch
    from synth.gen import make_predictor_layer
    from token_routing_speculation_amd.pipeline import PredictorPass

    N = cfg.N
    p = PredictorPass(N, cfg.d, cfg.E, cfg.K, cfg.hd)
    layers, truths, est = [], [], []
    fit_info = {}
    for l in range(cfg.L - 1):
        lay = make_predictor_layer(cfg, l)
        if args.fit and lay["estimator"]:
            fit_info[l] = fit_estimator(cfg, l, lay, args.fit_tokens, args.fit_ridge,
                                        time_oracle=not args.no_cpu_baseline and not fit_info)
        p.load(lay)
        p.truth = torch.empty((N, cfg.K), dtype=torch.int32, device="cuda")
        p.truth_step()
        layers.append(p.layer)
        truths.append(p.truth)
        est.append(bool(lay["estimator"]))
    torch.cuda.synchronize()
    return p, layers, truths, est, fit_info


def predictor_cpu_baseline(cfg, n_sample, min_seconds=10.0):
    """The oracle's prediction step (q_l, the next gate or the estimator,
    top-K, hits against the precomputed truth) on the first n_sample tokens of
    one benchmarked gate layer and one estimator layer, weighted to the
    sweep's mix of layers."""
    from synth import first_tokens
    from synth.gen import make_predictor_layer
    import oracle

    def one(layer, truth):
        q = oracle.route_qhidden(layer["r"], layer["dvec"], eps=layer["eps"])
        qb = oracle.round_bf16(q)
        if layer["estimator"]:
            lg = oracle.route_estimator(qb, layer["w1"], layer["b1"], layer["w2"], layer["b2"])
        else:
            lg = oracle.route_gate(qb, layer["w_next"])
        pred, _ = oracle.route_topk(lg, cfg.K, 1, 1)
        return oracle.hit_count(pred, truth)

    est_l, gate_l = cfg.est_layers[0], cfg.L - 2
    lays = {l: first_tokens(make_predictor_layer(cfg, l), n_sample) for l in (est_l, gate_l)}
    truths = {l: oracle.route_topk(oracle.route_gate(lay["s_next"], lay["w_next"]), cfg.K, 1, 1)[0]
              for l, lay in lays.items()}
    spent = {est_l: [0.0, 0], gate_l: [0.0, 0]}
    t_all = 0.0
    while t_all < min_seconds:
        for l in (est_l, gate_l):
            t0 = time.perf_counter()
            one(lays[l], truths[l])
            dt = time.perf_counter() - t0
            spent[l][0] += dt
            spent[l][1] += 1
            t_all += dt
    nl = cfg.L - 1
    ne = len(cfg.est_layers)
    per_layer = {l: spent[l][0] / spent[l][1] for l in spent}
    per_token = (ne * per_layer[est_l] + (nl - ne) * per_layer[gate_l]) / nl / n_sample
    threads = blas_threads()
    return {"value": 1.0 / per_token, "unit": "token-predictions/s", "cores": host_cores(),
            "blas_threads": threads, "kind": "oracle",
            "sample": f"the first {n_sample} benchmarked tokens of layer {gate_l} (gate) and layer "
                      f"{est_l} (estimator), {spent[gate_l][1]} + {spent[est_l][1]} passes, "
                      f"weighted {nl - ne}:{ne}; {t_all:.1f} s (float64 NumPy, matrix products on "
                      f"{threads} BLAS threads)"}


PREDICTOR_WORKLOAD = "qwen3-30b-a3b-shaped predictor"


def predictor_bench(args):
    """The q_l predictor sweep as its own bench line, with the oracle timed on
    the first tokens of the same layers."""
    from synth import get_config
    out = predictor_measure(args)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = predictor_cpu_baseline(get_config("qwen3"), min(args.cpu_sample, 1024))
    print(json.dumps(out), flush=True)
    return 0


def predictor_measure(args):
    """The q_l predictor of "Speculating Experts Accelerates Inference for
    Mixture-of-Experts" (technical summary items 2.A, 2.C and 4) over all
    source layers of the Qwen3-30B-A3B-shaped workload: per layer q_l = LN(d_l
    + r_l), the next gate on q_l (the MLP estimator on the early layers),
    top-K and the hit count against the next layer's true top-K (computed
    beforehand: it is layer l+1's own routing, not part of the prediction)."""
    import torch
    from synth import get_config
    from synth.gen import make_predictor_layer
    from token_routing_speculation_amd.pipeline import PredictorPass, capture_graph, to_device

    cfg = get_config("qwen3")
    torch.cuda.set_device(0)
    N = cfg.N
    p, layers, truths, est, fit_info = predictor_setup(cfg, args)

    def sweep(fused=True):
        for L_, T_ in zip(layers, truths):
            p.layer, p.truth = L_, T_
            p.step(fused)

    stream = torch.cuda.current_stream()
    K = args.steps
    # a plain copy of known size, untimed: the calibration kernel for the
    # FETCH_SIZE / WRITE_SIZE counters of a profiled run
    calib = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
    torch.empty_like(calib).copy_(calib)
    del calib

    def timed(fused):
        for _ in range(args.warmup):
            sweep(fused)
        torch.cuda.synchronize()
        graph = capture_graph(lambda: sweep(fused))
        for _ in range(args.warmup):
            graph.replay()
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(K + 1)]
        wall0 = time.perf_counter()
        ev[0].record(stream)
        for k in range(K):
            graph.replay()
            ev[k + 1].record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - wall0
        per = [ev[k].elapsed_time(ev[k + 1]) for k in range(K)]
        cold = cold_times(graph.replay, K) if fused else None
        del graph
        return ev[0].elapsed_time(ev[K]) / K, wall, per, cold

    ms_unfused, _, _, _ = timed(False)
    ms, wall, per_sweep, cold_sweep = timed(True)
    # per-stage times of one eager sweep, on an estimator layer and a gate layer
    def stage_times(i):
        p.layer, p.truth = layers[i], truths[i]
        from token_routing_speculation_amd import route_qhidden, route_estimator, route_gate, route_topk, hit_count
        L_ = p.layer
        e = [torch.cuda.Event(enable_timing=True) for _ in range(5)]
        tt = {"qhidden": [], "logits": [], "topk": [], "hits": []}
        for _ in range(10):
            e[0].record(stream)
            route_qhidden(L_["r"], L_["dvec"], eps=L_["eps"], q=p.q)
            e[1].record(stream)
            if L_["estimator"]:
                route_estimator(p.q, L_["w1"], L_["b1"], L_["w2"], L_["b2"], logits=p.logits, ws=p.ws)
            else:
                route_gate(p.q, L_["w_next"], logits=p.logits)
            e[2].record(stream)
            route_topk(p.logits, p.K, 1, 1, idx=p.pred, want_weights=False)
            e[3].record(stream)
            hit_count(p.pred, p.truth, p.hits)
            e[4].record(stream)
            torch.cuda.synchronize()
            for j, k_ in enumerate(tt):
                tt[k_].append(1e3 * e[j].elapsed_time(e[j + 1]))
        return {k_: round(float(np.median(v)), 2) for k_, v in tt.items()}

    def fused_stage_times(i):
        from token_routing_speculation_amd import route_qgate_topk_packed
        p.layer, p.truth = layers[i], truths[i]
        L_ = p.layer
        e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        tt = {"qgate_topk_hits": []}
        for _ in range(10):
            e[0].record(stream)
            route_qgate_topk_packed(L_["r"], L_["dvec"], L_["w_next_packed"], p.E, p.K,
                                    eps=L_["eps"], idx=p.pred, truth=p.truth, hits=p.hits)
            e[1].record(stream)
            torch.cuda.synchronize()
            for j, k_ in enumerate(tt):
                tt[k_].append(1e3 * e[j].elapsed_time(e[j + 1]))
        return {k_: round(float(np.median(v)), 2) for k_, v in tt.items()}
    st_est, st_gate = stage_times(0), stage_times(cfg.L - 2)
    st_fused = fused_stage_times(cfg.L - 2)

    def back_to_back_us(fn, reps=20):
        """Average duration of one launch over reps launches in a row."""
        for _ in range(3):
            fn()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return 1e3 * a.elapsed_time(b) / reps
    from token_routing_speculation_amd import route_qgate_topk, route_qgate_topk_packed
    Lg = layers[cfg.L - 2]
    qg_launch_us = back_to_back_us(
        lambda: route_qgate_topk_packed(Lg["r"], Lg["dvec"], Lg["w_next_packed"], p.E, p.K,
                                        eps=Lg["eps"], idx=p.pred, truth=p.truth, hits=p.hits))
    # the same call on the router's plain rows, for comparison
    qg_unpacked_us = back_to_back_us(
        lambda: route_qgate_topk(Lg["r"], Lg["dvec"], Lg["w_next"], p.K, eps=Lg["eps"], idx=p.pred,
                                 truth=p.truth, hits=p.hits))
    # the estimator's first product (with its bias, GELU and bf16 rounding)
    # beside the vendor GEMM on the same operands (torch.matmul, bf16 out, no
    # bias or GELU), both back to back on a resident q: context for
    # estimator_mfma_frac, not a part of the path
    from token_routing_speculation_amd import route_est_hidden
    Le = layers[0]
    h_est = torch.empty((N, cfg.hd), dtype=torch.bfloat16, device="cuda")
    w1_t = Le["w1"].view(torch.bfloat16).t().contiguous()
    q_bf = p.q.view(torch.bfloat16)
    est_first_us = back_to_back_us(lambda: route_est_hidden(p.q, Le["w1"], Le["b1"], h=h_est))
    vendor_first_us = back_to_back_us(lambda: torch.matmul(q_bf, w1_t, out=h_est))
    # q_l with the hidden layer in one kernel, as the fused sweep runs it
    from token_routing_speculation_amd import route_qest_hidden_packed
    q_hidden_us = (back_to_back_us(lambda: route_qest_hidden_packed(
        Le["r"], Le["dvec"], Le["w1_packed"], Le["b1"], cfg.hd, eps=Le["eps"], h=p.h))
        if "w1_packed" in Le else None)
    # one estimator layer's prediction: the one-kernel form the sweep runs
    # beside q_l + hidden layer, then output layer + top-K + hits
    from token_routing_speculation_amd import route_qest_topk_packed, route_est_out_topk_packed
    p.layer, p.truth = Le, truths[0]
    est_one_us = (back_to_back_us(lambda: route_qest_topk_packed(
        Le["r"], Le["dvec"], Le["w1_packed"], Le["b1"], cfg.hd, Le["w2_packed"], Le["b2"], p.E,
        p.K, eps=Le["eps"], idx=p.pred, truth=p.truth, hits=p.hits))
        if "w1_packed" in Le and cfg.hd in (512, 1024) and cfg.hd <= cfg.d else None)
    est_two_us = (back_to_back_us(lambda: (route_qest_hidden_packed(
        Le["r"], Le["dvec"], Le["w1_packed"], Le["b1"], cfg.hd, eps=Le["eps"], h=p.h),
        route_est_out_topk_packed(p.h, Le["w2_packed"], Le["b2"], p.E, p.K, idx=p.pred,
                                  truth=p.truth, hits=p.hits)))
        if "w1_packed" in Le and "w2_packed" in Le else None)
    del h_est, w1_t
    # hit rates per layer (one sweep from zeroed counters)
    p.hits.zero_()
    rates = []
    for L_, T_ in zip(layers, truths):
        before = int(p.hits.item())
        p.layer, p.truth = L_, T_
        p.step()
        rates.append((int(p.hits.item()) - before) / (N * cfg.K))
    # the same estimator layers predicted by the next gate on q_l instead
    gate_on_est = []
    for L_, T_, e_ in zip(layers, truths, est):
        if not e_:
            continue
        p.layer, p.truth = dict(L_, estimator=False), T_
        before = int(p.hits.item())
        p.step()
        gate_on_est.append((int(p.hits.item()) - before) / (N * cfg.K))
    nl = cfg.L - 1
    byt_gate = predictor_bytes(N, cfg.d, cfg.E, cfg.K, cfg.hd, False)
    byt_fused = predictor_bytes(N, cfg.d, cfg.E, cfg.K, cfg.hd, False, fused=True)
    byt_est = predictor_bytes(N, cfg.d, cfg.E, cfg.K, cfg.hd, True)
    byt_est_fused = predictor_bytes(N, cfg.d, cfg.E, cfg.K, cfg.hd, True, fused=True)
    ne = sum(est)
    total_unfused = ne * sum(byt_est.values()) + (nl - ne) * sum(byt_gate.values())
    total_bytes = ne * sum(byt_est_fused.values()) + (nl - ne) * sum(byt_fused.values())
    qg_us = qg_launch_us
    out = {
        "metric": "q_l expert-prediction throughput over all source layers (token-predictions/s)",
        "value": N * nl / (ms * 1e-3), "unit": "token-predictions/s", "n_gpus": 1,
        "steps": K, "warmup": args.warmup, "ms_per_step": ms, "launch": "hip graph replay",
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": PREDICTOR_WORKLOAD, "layers": nl, "N": N, "d": cfg.d,
                   "E": cfg.E, "K": cfg.K, "estimator_layers": list(cfg.est_layers), "hd": cfg.hd},
        "hbm_frac_sweep": total_bytes / (ms * 1e-3) / HBM_PEAK,
        "alg_bytes_sweep": total_bytes,
        "sweep_ms_p10_p50_p90": pct(per_sweep),
        "cold_sweep_ms_p10_p50_p90": pct(cold_sweep),
        "gate_layers": "route_qgate_topk with the hit count (q_l and the logits kept on chip)",
        "unfused": {"ms_per_step": ms_unfused, "value": N * nl / (ms_unfused * 1e-3),
                    "alg_bytes_sweep": total_unfused,
                    "hbm_frac_sweep": total_unfused / (ms_unfused * 1e-3) / HBM_PEAK,
                    "stages_us_gate_layer": st_gate},
        "stages_us_gate_layer": st_fused, "stages_us_estimator_layer": st_est,
        "qgate_topk_us_per_launch": qg_launch_us,
        "qgate_topk_unpacked_us_per_launch": qg_unpacked_us,
        "roofline": {"bound": "hbm", "kernel": "qgate_kernel<32, 2048, 1, true, true, 0> (route_qgate_topk_packed)",
                     "achieved": byt_fused["qgate_topk"] / (qg_us * 1e-6) / 1e9,
                     "peak": HBM_PEAK / 1e9, "unit": "GB/s",
                     "frac": byt_fused["qgate_topk"] / (qg_us * 1e-6) / HBM_PEAK,
                     "traffic": measured_traffic(PREDICTOR_WORKLOAD, QGATE_TRAFFIC_FILE,
                                                 QGATE_TRAFFIC_SOURCES)},
        "estimator_mfma_frac": (2.0 * N * cfg.d * cfg.hd + 2.0 * N * cfg.hd * cfg.E)
        / (st_est["logits"] * 1e-6) / MFMA_BF16_PEAK,
        "estimator_layer_us": {"one_kernel": est_one_us, "two_kernels": est_two_us,
                               "mfma_frac_one_kernel": (2.0 * N * cfg.d * cfg.hd
                                                        + 2.0 * N * cfg.hd * cfg.E)
                               / (est_one_us * 1e-6) / MFMA_BF16_PEAK if est_one_us else None},
        "estimator_first_product_us": {"route_est_hidden": est_first_us,
                                       "vendor_gemm_no_epilogue": vendor_first_us,
                                       "route_qest_hidden_packed_with_q_l": q_hidden_us,
                                       "mfma_frac": 2.0 * N * cfg.d * cfg.hd
                                       / (est_first_us * 1e-6) / MFMA_BF16_PEAK},
        "hit_rate_estimator_layers": float(np.mean([r for r, e_ in zip(rates, est) if e_])),
        "estimator_weights": ("fitted (ridge on a held-out batch of %d tokens)" % args.fit_tokens)
        if args.fit else "random (as drawn)",
        "fit": fit_info or None,
        "hit_rate_gate_layers": float(np.mean([r for r, e_ in zip(rates, est) if not e_])),
        "hit_rate_estimator_layers_by_gate_on_q": float(np.mean(gate_on_est)),
        "hit_rate_per_estimator_layer": [round(r, 4) for r, e_ in zip(rates, est) if e_],
        "wall_s_timed": wall,
    }
    return out


PCIE_PEAK = 64.0e9           # PCIe 5.0 x16 host link, bytes/s per direction (32 GT/s x 16 lanes)


def prefetch_bench(args):
    """Speculative expert prefetch ("Speculating Experts Accelerates Inference
    for Mixture-of-Experts", items 1, 2 and 4) for decoding a
    Qwen3-30B-A3B-shaped model whose expert weights sit in pinned host memory.
    For each decoded token and source layer l, layer l+1's experts are
    predicted from q_l (the predictor pass) and planned into C = K * batch
    staging slots. Four schedules of the transfers are timed per token:
      on_demand:   after layer l+1's routing, its true experts are copied
                   (prefetch_copy: the list stays on the GPU, which waits);
      speculative: the predicted experts are copied on a second stream by the
                   copy kernel, each layer's transfer planned while the one
                   before it still runs, so the transfers run back to back;
                   layer l+1 waits only for its copy (speculative execution
                   runs the prefetched experts);
      speculative_dma: the same through the DMA engines (prefetch_issue),
                   the list taken back to pinned host memory while the
                   previous transfer runs;
      prefetch_then_misses: the speculative schedule, then the true experts
                   that were not prefetched are copied after routing (no
                   speculative execution).
    The layers' own compute (attention, expert FFNs) is not built, so the
    schedules differ only by what they transfer and when. The overlap leg
    runs the N-row predictor sweep (compute) beside the transfers, through
    the DMA path and through the copy kernel."""
    import torch
    import token_routing_speculation_amd as tr
    from synth import get_config
    from token_routing_speculation_amd.pipeline import capture_graph

    cfg = get_config("qwen3")
    torch.cuda.set_device(0)
    E, K = cfg.E, cfg.K
    nl = cfg.L - 1
    B = args.prefetch_batch
    T = args.prefetch_tokens
    C = min(E, K * B)
    EB = 3 * cfg.d * cfg.ffn * 2
    W = min(2, T)                                  # warm-up tokens per schedule
    p, layers, truths, est, _ = predictor_setup(cfg, args)
    # layer l+1's predicted top-K for all N rows, from the predictor pass
    preds = []
    for L_, T_ in zip(layers, truths):
        p.layer, p.truth = L_, T_
        p.step()
        preds.append(p.pred.clone())
    torch.cuda.synchronize()
    assert T * B <= cfg.N
    bank = torch.empty((E, EB), dtype=torch.uint8, pin_memory=True)   # 1.2 GB, content irrelevant
    slots = torch.empty((2, C, EB), dtype=torch.uint8, device="cuda")
    miss_slots = torch.empty((E, EB), dtype=torch.uint8, device="cuda")
    lists = torch.empty((T, nl, C), dtype=torch.int32, device="cuda")
    lists_h = torch.empty((T, nl, C), dtype=torch.int32, pin_memory=True)
    nlists = torch.zeros((T, nl), dtype=torch.int32, device="cuda")
    tlists = torch.empty((T, nl, C), dtype=torch.int32, device="cuda")
    ntlists = torch.zeros((T, nl), dtype=torch.int32, device="cuda")
    misses = torch.empty((T, nl, E), dtype=torch.int32, device="cuda")
    nmisses = torch.zeros((T, nl), dtype=torch.int32, device="cuda")
    covered = torch.zeros((nl,), dtype=torch.int64, device="cuda")
    # the compute stream is a created one (default priority), made current, so
    # the schedules can also be captured as graphs on it
    torch.cuda.synchronize()
    comp = torch.cuda.Stream()
    torch.cuda.set_stream(comp)
    copy = torch.cuda.Stream()                     # default priority
    rows = lambda t: slice(t * B, (t + 1) * B)
    ev_plan = [torch.cuda.Event() for _ in range(nl)]
    ev_copy = [torch.cuda.Event() for _ in range(nl)]

    def token_on_demand(t):
        for l in range(nl):
            tr.prefetch_plan(truths[l][rows(t)], E, C, lst=tlists[t, l], nlist=ntlists[t, l:l + 1])
            tr.prefetch_copy(bank, tlists[t, l], slots[l % 2])

    def token_speculative(t, with_misses, dma=False):
        """Transfer l brings the experts predicted for layer l + 1 (from q_l).
        Transfer l + 1 is planned before the compute stream waits for
        transfer l: q_{l+1} exists once layer l has run, which needed only
        transfer l - 1. So the transfers queue back to back on the copy
        stream. The copy kernel keeps the list on the GPU; the DMA form
        (dma=True) takes it back to pinned host memory and issues
        prefetch_issue, while transfer l is still running."""
        def issue(l):
            tr.prefetch_plan(preds[l][rows(t)], E, C, lst=lists[t, l], nlist=nlists[t, l:l + 1])
            if dma:
                lists_h[t, l].copy_(lists[t, l], non_blocking=True)
            # one wait covers the plan and the slots: ev_plan[l] follows, on the
            # compute stream, the work of the layer that used slots[l % 2] last
            ev_plan[l].record(comp)
            copy.wait_event(ev_plan[l])
            if dma:
                ev_plan[l].synchronize()
                tr.prefetch_issue(bank, lists_h[t, l], slots[l % 2], stream=copy)
            else:
                with torch.cuda.stream(copy):
                    tr.prefetch_copy(bank, lists[t, l], slots[l % 2])
            ev_copy[l].record(copy)

        issue(0)
        for l in range(nl):
            if l + 1 < nl:
                issue(l + 1)
            # the layer these experts belong to starts once they are in
            comp.wait_event(ev_copy[l])
            tr.prefetch_coverage(truths[l][rows(t)], lists[t, l], E, covered[l:l + 1],
                                 miss=misses[t, l], nmiss=nmisses[t, l:l + 1])
            if with_misses:
                tr.prefetch_copy(bank, misses[t, l], miss_slots)

    def timed(fn):
        for t in range(W):
            fn(t)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(comp)
        for t in range(T):
            fn(t)
        e1.record(comp)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / T

    def timed_graph(fn):
        """Per-token time with each token's schedule captured once as a HIP
        graph (both streams; the cross-stream waits become graph edges)."""
        graphs = []
        for t in range(T):
            copy.wait_stream(comp)
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=comp):
                copy.wait_stream(comp)
                fn(t)
                comp.wait_stream(copy)
            graphs.append(g)
        torch.cuda.synchronize()
        for g in graphs[:W]:
            g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(comp)
        for g in graphs:
            g.replay()
        e1.record(comp)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / T

    ms_od = timed(token_on_demand)
    ms_sp_dma = timed(lambda t: token_speculative(t, False, dma=True))
    ms_sp = timed(lambda t: token_speculative(t, False))
    covered.zero_()
    ms_pm = timed(lambda t: token_speculative(t, True))
    ms_od_graph = timed_graph(token_on_demand)
    ms_sp_graph = timed_graph(lambda t: token_speculative(t, False))
    cov_by_layer = covered.cpu().numpy() / ((T + W) * B * K)
    byt_od = int(ntlists.sum()) * EB / T
    byt_sp = int(nlists.sum()) * EB / T
    byt_pm = byt_sp + int(nmisses.sum()) * EB / T

    # the copy kernel alone: one layer's C experts per launch, HIP events on its stream
    lst0, lst0_h = lists[0, 0], lists_h[0, 0]
    n_copied = int(nlists[0, 0])
    reps = args.steps
    for _ in range(3):
        tr.prefetch_copy(bank, lst0, slots[0])
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    ev[0].record(comp)
    for r in range(reps):
        tr.prefetch_copy(bank, lst0, slots[0])
        ev[r + 1].record(comp)
    torch.cuda.synchronize()
    copy_us = [1e3 * ev[r].elapsed_time(ev[r + 1]) for r in range(reps)]
    copy_gbs = n_copied * EB / (np.mean(copy_us) * 1e-6) / 1e9
    # the same layer's experts through the DMA engines
    for _ in range(3):
        tr.prefetch_issue(bank, lst0_h, slots[0])
    torch.cuda.synchronize()
    ev[0].record(comp)
    for r in range(reps):
        tr.prefetch_issue(bank, lst0_h, slots[0])
        ev[r + 1].record(comp)
    torch.cuda.synchronize()
    dma_us = [1e3 * ev[r].elapsed_time(ev[r + 1]) for r in range(reps)]
    dma_gbs = n_copied * EB / (np.mean(dma_us) * 1e-6) / 1e9

    # overlap: the N-row predictor sweep (compute) beside one layer's transfer, repeated
    def sweep():
        for L_, T_ in zip(layers, truths):
            p.layer, p.truth = L_, T_
            p.step()
    graph = capture_graph(sweep)
    graph.replay()
    torch.cuda.synchronize()
    n_ov = 5

    def sweeps_beside(xfer, n_x):
        """(ms per sweep, total transfer ms) with n_x transfers on the copy
        stream beside n_ov sweeps on the compute stream (n_x = 0: sweeps alone)."""
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        copy.wait_stream(comp)
        if n_x:
            c0.record(copy)
            with torch.cuda.stream(copy):
                for _ in range(n_x):
                    xfer()
            c1.record(copy)
        a.record(comp)
        for _ in range(n_ov):
            graph.replay()
        b.record(comp)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n_ov, (c0.elapsed_time(c1) if n_x else None)

    sweep_alone, _ = sweeps_beside(None, 0)
    n_x = max(1, int(round(n_ov * sweep_alone * 1e-3 / (np.mean(dma_us) * 1e-6))))
    overlap = {"sweep_ms_alone": sweep_alone, "transfers": n_x}
    for name, fn in (("dma", lambda: tr.prefetch_issue(bank, lst0_h, slots[1], stream=copy)),
                     ("kernel", lambda: tr.prefetch_copy(bank, lst0, slots[1]))):
        sw, xf = sweeps_beside(fn, n_x)
        overlap[f"sweep_ms_with_{name}"] = sw
        overlap[f"{name}_gbs_with_sweep"] = n_x * n_copied * EB / (xf * 1e-3) / 1e9

    out = {
        "metric": "speculative expert prefetch, host-to-GPU transfer rate (prefetch_issue, DMA)",
        "value": dma_gbs, "unit": "GB/s", "n_gpus": 1, "steps": reps, "warmup": 3,
        "ms_per_step": float(np.mean(dma_us)) / 1e3, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "u8", "data": "synthetic",
        "config": {"workload": "qwen3-30b-a3b-shaped decode, experts offloaded to pinned host memory",
                   "layers": nl, "E": E, "K": K, "batch": B, "slots": C, "expert_bytes": EB,
                   "tokens": T},
        "roofline": {"bound": "pcie", "kernel": "prefetch_copy_kernel", "achieved": copy_gbs,
                     "peak": PCIE_PEAK / 1e9, "unit": "GB/s", "frac": copy_gbs * 1e9 / PCIE_PEAK,
                     "traffic": None},
        "copy_kernel_us": {"mean": float(np.mean(copy_us)), "p50": float(np.median(copy_us)),
                           "experts": n_copied},
        "dma_us": {"mean": float(np.mean(dma_us)), "p50": float(np.median(dma_us))},
        "dma_frac_of_pcie": dma_gbs * 1e9 / PCIE_PEAK,
        "ms_per_token": {"on_demand": ms_od, "speculative": ms_sp, "speculative_dma": ms_sp_dma,
                         "prefetch_then_misses": ms_pm},
        "ms_per_token_graph": {"on_demand": ms_od_graph, "speculative": ms_sp_graph},
        "bytes_per_token": {"on_demand": byt_od, "speculative": byt_sp,
                            "prefetch_then_misses": byt_pm},
        "coverage": {"gate_layers": float(np.mean([c for c, e_ in zip(cov_by_layer, est) if not e_])),
                     "estimator_layers": float(np.mean([c for c, e_ in zip(cov_by_layer, est) if e_]))},
        "overlap": overlap,
    }
    if not args.no_cpu_baseline:
        from oracle import prefetch as opf
        lst_np = lst0_h.numpy().copy()
        bank_np = bank.numpy()
        sl = np.empty((C, EB), np.uint8)
        t0 = time.perf_counter()
        k = 0
        while time.perf_counter() - t0 < 3.0:
            sl = opf.prefetch_copy(bank_np, lst_np, sl)
            k += 1
        dt = time.perf_counter() - t0
        out["cpu_baseline"] = {"value": k * n_copied * EB / dt / 1e9, "unit": "GB/s", "cores": 1,
                               "kind": "oracle",
                               "sample": f"{k} copies of one layer's {n_copied} experts from the "
                                         "pinned bank into host slots (numpy)"}
    print(json.dumps(out), flush=True)
    return 0


def ceilings_bench(args):
    """Reference HBM rates of plain access patterns on this GPU, measured with
    torch's own kernels on 1 GiB buffers (no routing arithmetic): a pure read
    (a float32 sum), a pure write (a fill) and a copy. They bound the row
    movers from above (the combine is mostly reads, the dispatch mostly
    writes); the line reports each rate and its fraction of the 8 TB/s peak."""
    import torch
    torch.cuda.set_device(0)
    nbytes = 1 << 30
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    sink = torch.zeros((), dtype=torch.float32, device="cuda")
    pats = {"read": (lambda: torch.sum(src, dim=0, out=sink), nbytes),
            "write": (lambda: dst.fill_(7), nbytes),
            "copy": (lambda: dst.copy_(src), 2 * nbytes)}
    reps = max(args.steps, 5)
    out = {}
    for name, (fn, moved) in pats.items():
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        sec = a.elapsed_time(b) * 1e-3 / reps
        out[name] = {"gbs": moved / sec / 1e9, "frac": moved / sec / HBM_PEAK, "bytes": moved}
    line = {"metric": "HBM ceilings of plain access patterns (torch kernels, 1 GiB)",
            "value": out["read"]["gbs"], "unit": "GB/s", "n_gpus": 1, "steps": reps,
            "higher_is_better": True, "data": "synthetic", "patterns": out}
    print(json.dumps(line), flush=True)
    return 0


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="deepseek",
                    choices=["tiny", "mixtral", "deepseek", "foe", "qwen3"])
    ap.add_argument("--cpu-sample", type=int, default=4096, help="tokens in the oracle's timed sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-workloads", action="store_true",
                    help="deepseek: leave the other four workloads out of the line")
    ap.add_argument("--no-graph", action="store_true",
                    help="time eager launches only (default: the pass replayed as a HIP graph)")
    ap.add_argument("--eg", action="store_true",
                    help="measure the s-EG expert placement instead of the routing pass")
    ap.add_argument("--eg-iters", type=int, default=40)
    ap.add_argument("--eg-candidates", type=int, default=256)
    ap.add_argument("--eg-theta", type=float, default=0.0)
    ap.add_argument("--fit", action="store_true",
                    help="qwen3: fit the estimator layers' output weights before timing")
    ap.add_argument("--fit-tokens", type=int, default=32768)
    ap.add_argument("--fit-ridge", type=float, default=1e-3)
    ap.add_argument("--ceilings", action="store_true",
                    help="measure plain read / write / copy HBM rates with torch kernels")
    ap.add_argument("--prefetch", action="store_true",
                    help="qwen3: measure speculative expert prefetch from pinned host memory")
    ap.add_argument("--prefetch-tokens", type=int, default=16)
    ap.add_argument("--prefetch-batch", type=int, default=1)
    args = ap.parse_args(argv)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the routing path has no multi-GPU exchange "
              "(--gpus must be 1)", file=sys.stderr)
        return 2

    import torch
    from synth import make_config_inputs, get_config
    from token_routing_speculation_amd.pipeline import RoutePass, FoEPass, capture_graph

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 3
    if args.ceilings:
        return ceilings_bench(args)
    if args.prefetch:
        return prefetch_bench(args)
    if args.config == "qwen3":
        return predictor_bench(args)
    if args.eg:
        if args.config == "foe":
            print("--eg measures a routing workload (tiny, mixtral, deepseek)", file=sys.stderr)
            return 2
        return eg_bench(args)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 3
    torch.cuda.set_device(0)
    out, inp = route_measure(args, args.config)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(args.config, inp, min(args.cpu_sample, out["config"]["N"]))
    del inp
    if args.config == "deepseek" and not args.no_workloads:
        # the other four workloads, each timed the same way (no CPU baseline)
        wl = {}
        for name in ("tiny", "mixtral", "foe"):
            o, _ = route_measure(args, name)
            wl[name] = workload_summary(o)
            torch.cuda.empty_cache()
        o = predictor_measure(args)
        wl["qwen3"] = predictor_summary(o)
        out["workloads"] = wl
    print(json.dumps(out), flush=True)
    return 0


def workload_summary(o: dict) -> dict:
    """The figures of one routing or FoE workload kept in the default line."""
    return {"config": o["config"], "tokens_per_s": o["value"], "ms_per_pass": o["ms_per_step"],
            "warm_pass_ms_p50": o["pass_ms_p10_p50_p90"][1] if o["pass_ms_p10_p50_p90"] else None,
            "cold_pass_ms_p50": (o["cold_pass_ms_p10_p50_p90"][1]
                                 if o["cold_pass_ms_p10_p50_p90"] else None),
            "alg_bytes_pass": o["alg_bytes_pass"], "hbm_frac_pass": o["hbm_frac_pass"],
            "stages_us": o["stages_us"], "stage_hbm_frac": o["stage_hbm_frac"],
            "dominant_kernel": {k: o["roofline"][k] for k in ("kernel", "achieved", "unit", "frac")},
            "lar": o["lar"]}


def predictor_summary(o: dict) -> dict:
    """The figures of the q_l predictor sweep kept in the default line."""
    return {"config": o["config"], "token_predictions_per_s": o["value"],
            "ms_per_sweep": o["ms_per_step"],
            "sweep_ms_p10_p50_p90": o["sweep_ms_p10_p50_p90"],
            "cold_sweep_ms_p10_p50_p90": o["cold_sweep_ms_p10_p50_p90"],
            "alg_bytes_sweep": o["alg_bytes_sweep"], "hbm_frac_sweep": o["hbm_frac_sweep"],
            "dominant_kernel": {k: o["roofline"][k] for k in ("kernel", "achieved", "unit", "frac")},
            "estimator_mfma_frac": o["estimator_mfma_frac"],
            "estimator_layer_us": o["estimator_layer_us"],
            "hit_rate_gate_layers": o["hit_rate_gate_layers"],
            "hit_rate_estimator_layers": o["hit_rate_estimator_layers"]}


def route_measure(args, name):
    """One routing (tiny, mixtral, deepseek) or FoE workload: per-stage event
    times over eager passes, then the pass captured as a HIP graph and timed
    warm (replayed back to back) and cold (a 512 MiB read before each pass).
    Returns the bench line's fields (without the CPU baseline) and the
    inputs."""
    import torch
    from synth import make_config_inputs, get_config
    from token_routing_speculation_amd.pipeline import RoutePass, FoEPass, capture_graph

    cfg = get_config(name)
    inp = make_config_inputs(name)
    if name == "foe":
        p = FoEPass(inp)
        bytes_st = foe_bytes(cfg.N, cfg.d, cfg.E, cfg.K, cfg.H)
        conf = {"workload": "foe-grouped", "N": cfg.N, "d": cfg.d, "E": cfg.E, "H": cfg.H,
                "K": cfg.K, "G": cfg.G}
    else:
        p = RoutePass(inp)
        bytes_st = route_bytes(cfg.N, cfg.d, cfg.E, cfg.K, cfg.P, cfg.G, p.fallback, p.routed,
                               p.STAGES)
        conf = {"workload": ROUTE_WORKLOADS[name], "N": cfg.N, "d": cfg.d, "E": cfg.E,
                "K": cfg.K, "P": cfg.P, "G": cfg.G, "vocab": cfg.V,
                "fallback": "2-gram" if p.fallback else "none"}
    stages = p.STAGES
    stream = torch.cuda.current_stream()

    # a plain copy of known size, untimed: the calibration kernel for the
    # FETCH_SIZE / WRITE_SIZE counters of a profiled run
    calib = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
    calib_dst = torch.empty_like(calib)
    calib_dst.copy_(calib)
    del calib, calib_dst

    for _ in range(args.warmup):
        p.step()
    torch.cuda.synchronize()

    K = args.steps
    # eager steps, with events around every stage (per-stage and dominant-kernel times)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)] for _ in range(K)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record(stream)
    for k in range(K):
        for s, st in enumerate(stages):
            ev[k][s].record(stream)
            getattr(p, st)()
        ev[k][len(stages)].record(stream)
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_eager = t_start.elapsed_time(t_end) / K
    st_us = {st: 1e3 * sum(ev[k][s].elapsed_time(ev[k][s + 1]) for k in range(K)) / K
             for s, st in enumerate(stages)}
    ms = ms_eager
    per_pass = cold = None
    if not args.no_graph:
        # the same pass captured once and replayed: identical kernels, no
        # per-launch host gaps
        graph = capture_graph(p.step)
        for _ in range(args.warmup):
            graph.replay()
        torch.cuda.synchronize()
        ge = [torch.cuda.Event(enable_timing=True) for _ in range(K + 1)]
        wall0 = time.perf_counter()
        ge[0].record(stream)
        for k in range(K):
            graph.replay()
            ge[k + 1].record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - wall0
        ms = ge[0].elapsed_time(ge[K]) / K
        per_pass = [ge[k].elapsed_time(ge[k + 1]) for k in range(K)]
        cold = cold_times(graph.replay, K)
        del graph

    N = cfg.N
    tokens_per_s = N / (ms * 1e-3)
    total_bytes = sum(bytes_st.values())
    # the stage holding the router product
    gate_stage = next(g for g in ("gate", "srs_route", "predict_route", "predict_route_dispatch",
                                  "route") if g in st_us)
    # dominant kernel: the longest stage that is one launch
    fused_permute = cfg.E <= 16 and N * cfg.K <= 16384 and cfg.d <= 4096 and name != "foe"
    single = {"predict_route", "predict_route_dispatch", "srs_route", "combine", "route"}
    if fused_permute:
        single.add("permute")
    dom = max((st for st in stages if st in single), key=lambda st: st_us[st])
    dom_bytes = bytes_st[dom]
    achieved = dom_bytes / (st_us[dom] * 1e-6)
    small_route = cfg.E <= 64 and name != "foe"
    kernel_of = {
        "combine": ("combine_kernel (moe_combine)" if name == "foe"
                    else "combine_kernel (moe_combine_gather)"),
        "predict_route": "srs_route_kernel (srs_predict_route)",
        "predict_route_dispatch": "srs_route_kernel (srs_predict_route_dispatch)",
        "srs_route": ("srs_route_kernel (srs_route_sorted)" if small_route
                      else "srs_gate160_kernel (srs_route_sorted)"),
        "permute": "permute_fused (moe_permute)",
        "route": "srs_gate160_kernel (srs_route_grouped)",
    }
    out = {
        "metric": METRIC,
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "ms_per_step_eager": ms_eager,
        "launch": "eager" if args.no_graph else "hip graph replay",
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": conf,
        "hbm_frac_pass": total_bytes / (ms * 1e-3) / HBM_PEAK,
        "alg_bytes_pass": total_bytes,
        "pass_ms_p10_p50_p90": pct(per_pass) if per_pass else None,
        "cold_pass_ms_p10_p50_p90": pct(cold) if cold else None,
        "stages_us": {k: round(v, 2) for k, v in st_us.items()},
        "gate_stage": gate_stage,
        "gate_mfma_frac": 2.0 * N * cfg.d * cfg.E / (st_us[gate_stage] * 1e-6) / MFMA_BF16_PEAK,
        "stage_hbm_frac": {k: round(bytes_st[k] / (st_us[k] * 1e-6) / HBM_PEAK, 4) for k in stages},
        "roofline": {"bound": "hbm", "kernel": kernel_of[dom],
                     "achieved": achieved / 1e9, "peak": HBM_PEAK / 1e9, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK,
                     # the committed counter record is the combine's
                     "traffic": measured_traffic(conf["workload"]) if dom == "combine" else None},
        "lar": lar_rate(p, N * cfg.K),
        "wall_s_timed": wall,
    }
    del p
    return out, inp


def cold_times(replay, K):
    """Per-pass times (ms) of K replays, each after a 512 MiB read, so nothing
    a previous pass left in the 256 MB memory-side cache helps. The scrub only
    reads (the cache then holds clean lines): a writing scrub would charge the
    write-back of its own dirty lines to the pass."""
    import torch
    stream = torch.cuda.current_stream()
    scrub = torch.zeros(128 << 20, dtype=torch.float32, device="cuda")
    sink = torch.zeros((), dtype=torch.float32, device="cuda")
    for _ in range(3):
        torch.sum(scrub, dim=0, out=sink)
    ce = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(K)]
    for k in range(K):
        torch.sum(scrub, dim=0, out=sink)
        ce[k][0].record(stream)
        replay()
        ce[k][1].record(stream)
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in ce]


if __name__ == "__main__":
    sys.exit(main())
