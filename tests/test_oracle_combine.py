"""Pins for moe_combine: identity experts with normalised weights return the
input (plain and FoE cross-group sum), one-hot weights select one slot, the
out_row scatter, and a loop."""
import numpy as np

from oracle import moe_combine, moe_permute, route_topk
from oracle.bf16 import bf16_to_f64
from synth import to_bf16_bits


def test_identity_experts_return_input():
    rng = np.random.default_rng(0)
    N, E, K, d = 120, 8, 3, 16
    x = to_bf16_bits(rng.standard_normal((N, d)).astype(np.float32))
    idx, w = route_topk(rng.standard_normal((N, E)), K)
    r = moe_permute(idx, E, 1, x[None])
    out = moe_combine(r["disp"], w, r["slot_of_pair"])
    assert np.allclose(out, bf16_to_f64(x), rtol=1e-13, atol=1e-15)


def test_foe_identity_experts_sum_groups():
    rng = np.random.default_rng(1)
    N, E, H, K, d = 64, 16, 4, 8, 8
    x = to_bf16_bits(rng.standard_normal((H, N, d)).astype(np.float32))
    idx, w = route_topk(rng.standard_normal((N, E)), K, H)
    r = moe_permute(idx, E, H, x)
    out = moe_combine(r["disp"], w, r["slot_of_pair"])
    assert np.allclose(out, bf16_to_f64(x).sum(axis=0), rtol=1e-12, atol=1e-14)


def test_one_hot_weights_select_slot_and_out_row_scatter():
    rng = np.random.default_rng(2)
    N, K, d = 30, 4, 8
    y = to_bf16_bits(rng.standard_normal((N * K, d)).astype(np.float32))
    sop = rng.permutation(N * K)
    pick = rng.integers(0, K, N)
    w = np.zeros((N, K))
    w[np.arange(N), pick] = 1.0
    out_row = rng.permutation(N)
    out = moe_combine(y, w, sop, out_row)
    yd = bf16_to_f64(y)
    for j in range(N):
        assert np.array_equal(out[out_row[j]], yd[sop[j * K + pick[j]]])


def test_against_loop():
    rng = np.random.default_rng(3)
    N, K, d = 9, 3, 8
    y = to_bf16_bits(rng.standard_normal((N * K, d)).astype(np.float32))
    sop = rng.permutation(N * K)
    w = rng.random((N, K))
    out = moe_combine(y, w, sop)
    yd = bf16_to_f64(y)
    for j in range(N):
        acc = np.zeros(d)
        for k in range(K):
            acc += w[j, k] * yd[sop[j * K + k]]
        assert np.allclose(out[j], acc, rtol=1e-14)
