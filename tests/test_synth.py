"""The input generator: seeded determinism, shapes, and the distributions
of the recipe (Zipf ids, zero-sum split, per-id base independence)."""
import numpy as np

from synth import (make_route_inputs, make_foe_inputs, make_predictor_layer, get_config,
                   zipf_ids, from_bf16_bits, foe_row_cluster, default_expert_cluster)


def test_deterministic_and_shaped():
    a = make_route_inputs(256, 64, 8, 2, 2, 4, 1000, 5, ngram=True)
    b = make_route_inputs(256, 64, 8, 2, 2, 4, 1000, 5, ngram=True)
    for k in ("tok", "partials", "w", "lut", "conf", "ngram", "prev2", "prev1"):
        assert np.array_equal(a[k], b[k]), k
    assert a["partials"].shape == (2, 256, 64) and a["partials"].dtype == np.uint16
    assert a["w"].shape == (8, 64) and a["tok"].dtype == np.int32
    assert a["ngram"].shape == (4, 4) and a["lut"].max() < 4


def test_zero_sum_split_reconstructs_hidden():
    a = make_route_inputs(512, 128, 4, 2, 2, 2, 50, 3, noise=0.0)
    s = from_bf16_bits(a["partials"]).astype(np.float64).sum(axis=0)
    where = np.searchsorted(a["ids_present"], a["tok"])
    base = from_bf16_bits(a["base_present"]).astype(np.float64)[where]
    # each partial carries one bf16 rounding of a value of size ~ 1
    assert np.max(np.abs(s - base)) < 0.05
    assert np.corrcoef(s.ravel(), base.ravel())[0, 1] > 0.999


def test_base_rows_independent_of_sample():
    a = make_route_inputs(64, 32, 4, 2, 1, 2, 30, 9)
    b = make_route_inputs(300, 32, 4, 2, 1, 2, 30, 9)
    common = np.intersect1d(a["ids_present"], b["ids_present"])
    ia = np.searchsorted(a["ids_present"], common)
    ib = np.searchsorted(b["ids_present"], common)
    assert np.array_equal(a["base_present"][ia], b["base_present"][ib])


def test_zipf_rank_frequency():
    ids = zipf_ids(np.random.default_rng(0), 400000, 1000, 1.1)
    c = np.bincount(ids, minlength=1000).astype(np.float64)
    r = np.arange(1, 1001)
    slope = np.polyfit(np.log(r[:100]), np.log(c[:100]), 1)[0]
    assert abs(slope + 1.1) < 0.05


def test_foe_and_predictor_shapes():
    f = make_foe_inputs(128, 32, 16, 4, 8, 8, 100, 1)
    assert f["x"].shape == (4, 128, 32) and f["row_cluster"].shape == (512,)
    assert np.array_equal(f["row_cluster"][:8], [0, 2, 4, 6, 1, 3, 5, 7])
    assert np.array_equal(foe_row_cluster(3, 4, 2), [0, 0, 1, 1] * 3)
    assert np.array_equal(default_expert_cluster(8, 4), [0, 0, 1, 1, 2, 2, 3, 3])
    cfg = get_config("qwen3")
    lay = make_predictor_layer(cfg, 2, N=16)
    assert lay["estimator"] and lay["w1"].shape == (512, 2048) and lay["w2"].shape == (128, 512)
    lay = make_predictor_layer(cfg, 10, N=16)
    assert not lay["estimator"] and lay["s_next"].shape == (16, 2048)


def test_first_tokens_cuts_every_per_token_array():
    """first_tokens keeps the first n tokens of a drawn batch: the same ids,
    partial rows, previous clusters and FoE rows, and every table unchanged."""
    from synth import first_tokens, make_config_inputs
    a = make_config_inputs("tiny", N=64)
    b = first_tokens(a, 10)
    assert b["N"] == 10 and np.array_equal(b["tok"], a["tok"][:10])
    assert np.array_equal(b["partials"], a["partials"][:, :10]) and b["partials"].flags.c_contiguous
    assert b["lut"] is a["lut"] and b["w"] is a["w"]
    f = make_config_inputs("foe", N=32)
    g = first_tokens(f, 5)
    assert np.array_equal(g["x"], f["x"][:, :5]) and len(g["row_cluster"]) == 5 * f["H"]
    assert np.array_equal(g["row_cluster"], f["row_cluster"][:20])
    assert first_tokens(a, 1000)["N"] == 64
