"""Pins for route_qhidden (torch layer_norm in float64, moment identities),
the estimator (math.erf GELU, torch linear in float64) and hit_count."""
import math

import numpy as np
import torch
import torch.nn.functional as F

from oracle import route_qhidden, route_estimator, gelu_erf, hit_count, route_topk
from oracle.bf16 import bf16_to_f64
from synth import to_bf16_bits


def test_layernorm_against_torch():
    rng = np.random.default_rng(0)
    N, d = 40, 96
    r = to_bf16_bits(rng.standard_normal((N, d)).astype(np.float32))
    dv = rng.standard_normal(d).astype(np.float32) * 0.3
    g = rng.standard_normal(d).astype(np.float32)
    b = rng.standard_normal(d).astype(np.float32)
    q = route_qhidden(r, dv, g, b, 1e-5)
    v = torch.from_numpy(bf16_to_f64(r) + dv.astype(np.float64))
    ref = F.layer_norm(v, (d,), torch.from_numpy(g.astype(np.float64)),
                       torch.from_numpy(b.astype(np.float64)), 1e-5).numpy()
    assert np.allclose(q, ref, rtol=1e-12, atol=1e-12)


def test_layernorm_moments():
    rng = np.random.default_rng(1)
    N, d, eps = 30, 2048, 1e-5
    r = to_bf16_bits((rng.standard_normal((N, d)) * 0.01).astype(np.float32))
    dv = np.zeros(d, dtype=np.float32)
    q = route_qhidden(r, dv, eps=eps)
    v = bf16_to_f64(r)
    s2 = v.var(axis=1)
    assert np.allclose(q.mean(axis=1), 0.0, atol=1e-12)
    assert np.allclose(q.var(axis=1), s2 / (s2 + eps), rtol=1e-10)


def test_gelu_against_math_erf_and_torch():
    x = np.linspace(-8, 8, 2001)
    want = np.array([0.5 * t * (1 + math.erf(t / math.sqrt(2))) for t in x])
    assert np.allclose(gelu_erf(x), want, rtol=1e-14, atol=1e-15)
    assert np.allclose(gelu_erf(x), F.gelu(torch.from_numpy(x)).numpy(), rtol=1e-13, atol=1e-15)


def test_estimator_against_torch_linear():
    rng = np.random.default_rng(2)
    N, d, hd, E = 16, 64, 32, 24
    q = to_bf16_bits(rng.standard_normal((N, d)).astype(np.float32))
    w1 = to_bf16_bits((rng.standard_normal((hd, d)) / 8).astype(np.float32))
    w2 = to_bf16_bits((rng.standard_normal((E, hd)) / 6).astype(np.float32))
    b1 = rng.standard_normal(hd)
    b2 = rng.standard_normal(E)
    got = route_estimator(q, w1, b1, w2, b2)
    t = lambda a: torch.from_numpy(bf16_to_f64(a))
    h = F.gelu(F.linear(t(q), t(w1), torch.from_numpy(b1)))
    ref = F.linear(h, t(w2), torch.from_numpy(b2)).numpy()
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_hit_count_cases():
    rng = np.random.default_rng(3)
    N, E, K = 4000, 128, 8
    a, _ = route_topk(rng.standard_normal((N, E)), K)
    b, _ = route_topk(rng.standard_normal((N, E)), K)
    assert hit_count(a, a) == N * K
    assert hit_count(a, np.where(a < E // 2, a + E, a + 2 * E)) == 0
    h = hit_count(a, b)
    p = K / E
    assert abs(h - N * K * p) < 4 * math.sqrt(N * K * p * (1 - p))
    # duplicates count once, as a set intersection
    assert hit_count(np.array([[1, 1, 2]]), np.array([[1, 3, 4]])) == 1
