"""Pins for route_predict: table lookup, 2-gram fallback, threshold edge."""
import numpy as np
import pytest

from oracle import route_predict


def _inputs(n=500, V=97, G=8, seed=0):
    rng = np.random.default_rng(seed)
    return dict(tok=rng.integers(0, V, n).astype(np.int32),
                lut=rng.integers(0, G, V, dtype=np.uint8),
                conf=rng.integers(0, 256, V, dtype=np.uint8),
                prev2=rng.integers(0, G, n, dtype=np.uint8),
                prev1=rng.integers(0, G, n, dtype=np.uint8),
                ngram=rng.integers(0, G, (G, G), dtype=np.uint8))


def test_lookup_only_is_take():
    a = _inputs()
    assert np.array_equal(route_predict(a["tok"], a["lut"]), np.take(a["lut"], a["tok"]))


def test_confident_table_never_falls_back():
    a = _inputs()
    conf = np.full_like(a["conf"], 128)
    got = route_predict(a["tok"], a["lut"], conf, a["prev2"], a["prev1"], a["ngram"], 128)
    assert np.array_equal(got, np.take(a["lut"], a["tok"]))


def test_unconfident_table_always_falls_back():
    a = _inputs()
    conf = np.full_like(a["conf"], 127)
    got = route_predict(a["tok"], a["lut"], conf, a["prev2"], a["prev1"], a["ngram"], 128)
    want = a["ngram"][a["prev2"].astype(int), a["prev1"].astype(int)]
    assert np.array_equal(got, want)


def test_mixed_against_loop():
    a = _inputs(seed=3)
    got = route_predict(a["tok"], a["lut"], a["conf"], a["prev2"], a["prev1"], a["ngram"], 128)
    table = {v: int(a["lut"][v]) for v in range(len(a["lut"]))}
    for i, t in enumerate(a["tok"].tolist()):
        if int(a["conf"][t]) / 255.0 < 0.5:
            want = int(a["ngram"][a["prev2"][i]][a["prev1"][i]])
        else:
            want = table[t]
        assert got[i] == want


def test_out_of_vocabulary_raises():
    a = _inputs()
    tok = a["tok"].copy()
    tok[3] = len(a["lut"])
    with pytest.raises(ValueError):
        route_predict(tok, a["lut"])
