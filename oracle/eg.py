"""Plain definitions of speculative expert grouping (s-EG) (oracle).

TEST INFRASTRUCTURE ONLY (see the package docstring).

"Speculative MoE" notes, section 3.2 (s-EG: experts that the same tokens
activate together are placed in the same cluster, offline, and the gate's
columns are permuted so the move is transparent) and section 4.2 (balanced
token-expert co-clustering: a 0-1 program over token and expert cluster
assignments whose objective is a theta-weighted sum of the token-load
imbalance across clusters and the token-expert activations that cross
clusters, with every token and expert in exactly one cluster and the same
number of experts per cluster; solved approximately by a two-stage
cross-entropy optimisation).

The pages give the objective's two terms and the constraints, not their
normalisation nor the steps of the cross-entropy method. The readings taken
here (each also listed in the design notes):

* Profile: counts[u][e] = how often token id u (a row of the present-id
  table) routed to expert e in a profiled batch; freq[u] = how often u
  occurred.
* Stage 2 (tokens, given an expert placement x): every token goes to the
  cluster holding most of its activations, S[u][g] = sum of counts[u][e]
  over the experts e with x[e] = g, lowest g on ties. That is the token ->
  cluster table the routing path already builds.
* Objective of a placement (lower is better):
      J = (1 - theta) * (1 - local / T) + theta * (G * max_g L[g] / F - 1)
  with local = sum_u max_g S[u][g], T = sum of all counts, L[g] = sum of
  freq[u] over the tokens sent to g, F = sum of freq.
* Stage 1 (experts) by the cross-entropy method: a probability table P[e][g]
  (uniform to start); each iteration draws B placements, expert by expert in
  index order, cluster g with probability proportional to P[e][g] among the
  clusters that still have room (E / G experts each); keeps the
  ceil(rho * B) placements of lowest J (ties to the lower candidate index);
  moves P to alpha * (elite frequency) + (1 - alpha) * P; remembers the best
  placement seen (strict improvement).
* Random numbers: the counter-based form of SplitMix64 (Steele, Lea and
  Flood; Vigna's reference generator): output n of a generator seeded with
  s is mix(s + n * 0x9E3779B97F4A7C15) mod 2^64. Draw (iteration t,
  candidate b, expert e) uses n = (t * B + b) * E + e + 1, and becomes a
  double in [0, 1) from its top 53 bits.

Integer results are exact (int64). Floating point is float64 in the order
written, which the kernels follow operation for operation.
"""

from __future__ import annotations

import numpy as np

MASK64 = (1 << 64) - 1
GAMMA = 0x9E3779B97F4A7C15


def splitmix64(seed: int, n: int) -> int:
    """Output n (n >= 1) of SplitMix64 started from state ``seed``."""
    z = (seed + n * GAMMA) & MASK64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & MASK64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & MASK64
    return z ^ (z >> 31)


def uniform01(seed: int, n: int) -> float:
    """Draw n as a double in [0, 1): the top 53 bits of the output."""
    return (splitmix64(seed, n) >> 11) * (1.0 / (1 << 53))


def draw_index(t: int, b: int, e: int, B: int, E: int) -> int:
    return (t * B + b) * E + e + 1


def coact_profile(tok, idx, row_of_id, U, E):
    """counts[U][E] and freq[U] of a routed batch (tok[n], idx[n][K])."""
    tok = np.asarray(tok, dtype=np.int64)
    idx = np.asarray(idx, dtype=np.int64)
    rows = np.asarray(row_of_id, dtype=np.int64)[tok]
    if (rows < 0).any() or (idx < 0).any() or (idx >= E).any():
        raise ValueError("token without a profile row, or expert out of range")
    counts = np.zeros((U, E), dtype=np.int64)
    freq = np.zeros(U, dtype=np.int64)
    for i in range(len(tok)):
        freq[rows[i]] += 1
        for e in idx[i]:
            counts[rows[i], e] += 1
    return counts, freq


def eg_score(counts, freq, place, G):
    """For each placement place[b][E]: local[b] and load[b][G] (int64)."""
    counts = np.asarray(counts, dtype=np.int64)
    freq = np.asarray(freq, dtype=np.int64)
    place = np.asarray(place, dtype=np.int64)
    B = place.shape[0]
    local = np.zeros(B, dtype=np.int64)
    load = np.zeros((B, G), dtype=np.int64)
    for b in range(B):
        # S[u][g]: token u's activations of the experts placed in cluster g
        S = np.stack([counts[:, place[b] == g].sum(axis=1) for g in range(G)], axis=1)
        best = np.argmax(S, axis=1)               # first maximum: lowest g on ties
        local[b] = S[np.arange(S.shape[0]), best].sum()
        load[b] = np.bincount(best, weights=freq, minlength=G).astype(np.int64)
    return local, load


def eg_objective(local, load, T, F, G, theta):
    """J[b] of each scored placement (float64, the kernel's order)."""
    local = np.asarray(local, dtype=np.int64)
    load = np.asarray(load, dtype=np.int64)
    r = 1.0 - local.astype(np.float64) / float(T)
    bal = float(G) * load.max(axis=1).astype(np.float64) / float(F) - 1.0
    return (1.0 - theta) * r + theta * bal


def eg_sample(P, B, G, seed, t):
    """B placements [B][E] (uint8) drawn from P[E][G] under equal capacity."""
    P = np.asarray(P, dtype=np.float64)
    E = P.shape[0]
    cap0 = E // G
    place = np.zeros((B, E), dtype=np.uint8)
    for b in range(B):
        cap = [cap0] * G
        for e in range(E):
            w = [P[e, g] if cap[g] > 0 else 0.0 for g in range(G)]
            W = 0.0
            for g in range(G):
                W = W + w[g]
            target = uniform01(seed, draw_index(t, b, e, B, E)) * W
            pick = -1
            c = 0.0
            for g in range(G):
                c = c + w[g]
                if w[g] > 0.0 and c > target:
                    pick = g
                    break
            if pick < 0:
                # rounding left the target at the top: the last open cluster
                # of positive weight; no weight left at all: the first open one
                if W > 0.0:
                    pick = max(g for g in range(G) if w[g] > 0.0)
                else:
                    pick = min(g for g in range(G) if cap[g] > 0)
            place[b, e] = pick
            cap[pick] -= 1
    return place


def eg_update(P, place, J, n_elite, alpha, best_J, best_place):
    """One cross-entropy update: (P', best_J', best_place')."""
    P = np.asarray(P, dtype=np.float64)
    place = np.asarray(place, dtype=np.int64)
    J = np.asarray(J, dtype=np.float64)
    B, E = place.shape
    G = P.shape[1]
    rank = np.empty(B, dtype=np.int64)
    for b in range(B):
        rank[b] = int((J < J[b]).sum() + (J[:b] == J[b]).sum())
    elite = rank < n_elite
    Pn = np.empty_like(P)
    for e in range(E):
        for g in range(G):
            cnt = int((place[elite, e] == g).sum())
            Pn[e, g] = alpha * (cnt / float(n_elite)) + (1.0 - alpha) * P[e, g]
    bmin = int(np.argmin(rank))
    if J[bmin] < best_J:
        return Pn, float(J[bmin]), place[bmin].astype(np.uint8).copy()
    return Pn, best_J, np.asarray(best_place, dtype=np.uint8).copy()


def ceo_place(counts, freq, G, theta=0.0, B=256, iters=30, rho=0.1, alpha=0.7, seed=0):
    """Cross-entropy placement of E experts in G equal clusters.

    Returns (best_place[E] uint8, best_J, P[E][G], history of best_J).
    """
    counts = np.asarray(counts, dtype=np.int64)
    freq = np.asarray(freq, dtype=np.int64)
    E = counts.shape[1]
    if E % G:
        raise ValueError("E must be a multiple of G")
    T = int(counts.sum())
    F = int(freq.sum())
    n_elite = max(1, int(np.ceil(rho * B)))
    P = np.full((E, G), 1.0 / G)
    best_J = np.inf
    best_place = np.zeros(E, dtype=np.uint8)
    hist = []
    for t in range(iters):
        place = eg_sample(P, B, G, seed, t)
        local, load = eg_score(counts, freq, place, G)
        J = eg_objective(local, load, T, F, G, theta)
        P, best_J, best_place = eg_update(P, place, J, n_elite, alpha, best_J, best_place)
        hist.append(best_J)
    return best_place, best_J, P, hist
