"""Pins of the estimator-fit oracle ("Speculating Experts Accelerates
Inference for Mixture-of-Experts", item 2.C): closed forms on orthogonal
(Hadamard) features, exact recovery of a linear target, the Gram matrix's
structure, and the ridge residual identity."""

import numpy as np
import pytest

from oracle import estfit
from oracle.bf16 import round_bf16, bf16_to_f64


def _hadamard(n):
    H = np.array([[1.0]])
    while H.shape[0] < n:
        H = np.block([[H, H], [H, -H]])
    return H


def test_orthogonal_features_closed_form():
    n, hd, E, ridge = 64, 31, 5, 0.25
    Had = _hadamard(n)                     # columns orthogonal, column 0 all ones
    h = round_bf16(Had[:, 1:hd + 1])       # +-1: exact in bf16
    y = np.random.default_rng(1).standard_normal((n, E))
    G, R = estfit.est_gram(h, y)
    assert np.array_equal(G, n * np.eye(hd + 1))
    Wp = estfit.est_solve(G, R, ridge)
    # G = n I: W' = R / (n + ridge * n)
    assert np.allclose(Wp, R / (n * (1.0 + ridge)), rtol=1e-13, atol=0)


def test_recovers_an_exact_linear_target():
    rng = np.random.default_rng(2)
    n, hd, E = 400, 24, 7
    h = round_bf16(rng.standard_normal((n, hd)))
    Wt = rng.standard_normal((hd + 1, E))
    Hp = np.concatenate([bf16_to_f64(h), np.ones((n, 1))], axis=1)
    y = Hp @ Wt
    w2, b2, Wp = estfit.est_fit(h, y, 1e-14)
    assert np.allclose(Wp, Wt, rtol=0, atol=1e-7)
    assert np.array_equal(w2, round_bf16(Wp[:-1].T))
    assert np.array_equal(b2, Wp[-1].astype(np.float32))


def test_gram_structure():
    rng = np.random.default_rng(3)
    n, hd, E = 77, 10, 3
    h = round_bf16(rng.standard_normal((n, hd)))
    y = rng.standard_normal((n, E)).astype(np.float32)
    G, R = estfit.est_gram(h, y)
    H = bf16_to_f64(h)
    assert np.array_equal(G, G.T) and G[-1, -1] == n
    assert np.allclose(G[-1, :-1], H.sum(axis=0), rtol=1e-15)
    assert np.allclose(R[-1], y.astype(np.float64).sum(axis=0), rtol=1e-12)
    assert np.linalg.eigvalsh(G).min() > -1e-9


@pytest.mark.parametrize("ridge", [1e-3, 0.1])
def test_ridge_residual_identity(ridge):
    rng = np.random.default_rng(4)
    n, hd, E = 300, 16, 4
    h = round_bf16(rng.standard_normal((n, hd)))
    y = rng.standard_normal((n, E))
    G, R = estfit.est_gram(h, y)
    Wp = estfit.est_solve(G, R, ridge)
    Hp = np.concatenate([bf16_to_f64(h), np.ones((n, 1))], axis=1)
    lam = ridge * np.trace(G) / (hd + 1)
    # normal equations through the residual: H'^T (Y - H' W') = lambda W'
    assert np.allclose(Hp.T @ (y - Hp @ Wp), lam * Wp, rtol=1e-9, atol=1e-9)
