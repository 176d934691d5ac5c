"""Pins for route_gate: one-hot closed forms (catch transposes), integer
exact products against a Python loop, and the binary32 error bound."""
import numpy as np
import torch

from oracle import route_gate
from oracle.bf16 import bf16_to_f64
from synth import to_bf16_bits


def test_one_hot_weight_rows_pick_columns():
    N, d, E = 7, 24, 5
    x = to_bf16_bits(np.random.default_rng(0).standard_normal((N, d)).astype(np.float32))
    cols = [3, 0, 23, 11, 3]
    w = np.zeros((E, d), dtype=np.float32)
    for e, c in enumerate(cols):
        w[e, c] = 1.0
    g = route_gate(x, to_bf16_bits(w))
    assert g.shape == (N, E)
    assert np.array_equal(g, bf16_to_f64(x)[:, cols])


def test_one_hot_token_rows_pick_weight_columns():
    N, d, E = 6, 16, 9
    w = to_bf16_bits(np.random.default_rng(1).standard_normal((E, d)).astype(np.float32))
    cols = [0, 15, 7, 7, 2, 9]
    x = np.zeros((N, d), dtype=np.float32)
    for i, c in enumerate(cols):
        x[i, c] = 2.0
    g = route_gate(to_bf16_bits(x), w)
    assert np.array_equal(g, 2.0 * bf16_to_f64(w)[:, cols].T)


def test_integer_operands_against_loop():
    rng = np.random.default_rng(2)
    N, d, E = 5, 12, 3
    xi = rng.integers(-8, 9, (N, d))
    wi = rng.integers(-8, 9, (E, d))
    g = route_gate(to_bf16_bits(xi.astype(np.float32)), to_bf16_bits(wi.astype(np.float32)))
    for i in range(N):
        for e in range(E):
            assert g[i, e] == sum(int(xi[i, k]) * int(wi[e, k]) for k in range(d))


def test_binary32_matmul_within_bound():
    rng = np.random.default_rng(3)
    x = to_bf16_bits(rng.standard_normal((64, 256)).astype(np.float32))
    w = to_bf16_bits((rng.standard_normal((16, 256)) / 16).astype(np.float32))
    g = route_gate(x, w)
    xt = torch.from_numpy(x.view(np.int16).copy()).view(torch.bfloat16).float()
    wt = torch.from_numpy(w.view(np.int16).copy()).view(torch.bfloat16).float()
    ref = (xt @ wt.T).double().numpy()
    assert np.max(np.abs(g - ref)) < 1e-4
