"""Plain definition of fitting the lightweight estimator (oracle).

TEST INFRASTRUCTURE ONLY (see the package docstring).

"Speculating Experts Accelerates Inference for Mixture-of-Experts", technical
summary item 2.C: a shallow network trained to predict the next layer's
router logits from q_l, used on the layers where q_l alone predicts poorly
(item 4: a few million training tokens reach high hit rates). The page does
not give the training procedure. The reading taken here: the hidden layer
GELU(q W1^T + b1) stays as drawn (random features, as the estimator computes
them, rounded to bf16), and the output layer is the ridge-regression fit of
the true logits Y on those features with a bias column:

    H' = [H | 1],   (H'^T H' + lambda I) W' = H'^T Y,
    lambda = ridge * trace(H'^T H') / (hd + 1),
    W2 = W'[:hd]^T (rounded to bf16),   b2 = W'[hd].

Float64 throughout (the features are bf16, so every product H'^T H' and
H'^T Y forms exactly); numpy's LAPACK solve serves as the linear solve.
"""

from __future__ import annotations

import numpy as np

from .bf16 import bf16_to_f64, round_bf16


def est_gram(h_bits, y):
    """G = H'^T H' and R = H'^T Y for bf16 features h [n][hd] and float logits y [n][E]."""
    H = bf16_to_f64(h_bits)
    n = H.shape[0]
    Hp = np.concatenate([H, np.ones((n, 1))], axis=1)
    Y = np.asarray(y, dtype=np.float64)
    return Hp.T @ Hp, Hp.T @ Y


def est_solve(G, R, ridge):
    """W' of (G + lambda I) W' = R, lambda = ridge * trace(G) / m."""
    G = np.asarray(G, dtype=np.float64)
    m = G.shape[0]
    lam = ridge * np.trace(G) / m
    return np.linalg.solve(G + lam * np.eye(m), np.asarray(R, dtype=np.float64))


def est_weights(Wp):
    """(w2 bf16 bits [E][hd], b2 float32 [E]) from W' [hd + 1][E]."""
    Wp = np.asarray(Wp, dtype=np.float64)
    return round_bf16(Wp[:-1].T.copy()), Wp[-1].astype(np.float32)


def est_fit(h_bits, y, ridge):
    """The whole fit: features and targets -> (w2 bits, b2, W')."""
    G, R = est_gram(h_bits, y)
    Wp = est_solve(G, R, ridge)
    w2, b2 = est_weights(Wp)
    return w2, b2, Wp
