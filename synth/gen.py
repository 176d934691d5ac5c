"""Seeded generators for every input of the routing path.

Recipe (all streams are ``numpy.random.default_rng([seed, stream, ...])``):

* token ids: truncated Zipf(s) over the vocabulary, P(id = r-1) ~ r**-s for
  r = 1..V, drawn by inverse CDF on a float64 cumulative table (stream 0);
* per-id base vector ``base[v] ~ N(0, 1)^d`` from its own counter-keyed stream
  ``[seed, 1, v]``, so a row does not depend on sampling order;
* hidden = base[id] + noise * N(0, 1) (stream 2), float32;
* P tensor-parallel partials by a zero-sum split:
  ``part_p = bf16(hidden / P + u_p - mean_p(u))`` with ``u ~ N(0, 0.25)``
  (stream 3). The FoE per-group activations use the same split with P = H;
* gate weights ``W ~ N(0, 1/d)`` in bf16 (stream 4);
* token -> cluster table: uniform bytes in [0, G) (stream 5); in "routing"
  mode the caller replaces the entries of the ids that occur with the table
  builder's output (argmax cluster of each id's noiseless routing), the rest
  stay filler that the path never reads;
* confidence bytes uniform in [0, 256) as filler (stream 5), 2-gram table
  ``A[G][G]`` uniform in [0, G) (stream 6), previous-layer clusters
  ``prev2, prev1`` uniform in [0, G) (stream 7).

Another batch of the same model (``sample`` > 0, for profiling) keys the
token, noise and split streams as ``[seed, stream, sample]``.

Variance convention: ``N(0, v)`` names the variance, so W has std 1/sqrt(d).
"""

from __future__ import annotations

import numpy as np
import torch

from .configs import RouteConfig, FoEConfig, PredictorConfig, get_config


def _rng(*key):
    return np.random.default_rng(list(key))


def to_bf16_bits(x) -> np.ndarray:
    """float array -> uint16 bf16 bit patterns (round to nearest even)."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def from_bf16_bits(u) -> np.ndarray:
    """uint16 bf16 bit patterns -> float32 (exact)."""
    u = np.ascontiguousarray(u, dtype=np.uint16)
    return (u.astype(np.uint32) << 16).view(np.float32)


def zipf_ids(rng, n: int, vocab: int, s: float = 1.1) -> np.ndarray:
    """Truncated Zipf(s) sample of n ids in [0, vocab), by inverse CDF."""
    r = np.arange(1, vocab + 1, dtype=np.float64)
    cdf = np.cumsum(r ** (-s))
    cdf /= cdf[-1]
    u = rng.random(n)
    ids = np.searchsorted(cdf, u, side="right")
    return np.minimum(ids, vocab - 1).astype(np.int32)


def _base_rows(seed: int, ids: np.ndarray, d: int) -> np.ndarray:
    out = np.empty((len(ids), d), dtype=np.float32)
    for j, v in enumerate(ids):
        out[j] = _rng(seed, 1, int(v)).standard_normal(d, dtype=np.float32)
    return out


def _zero_sum_split(rng, hidden: np.ndarray, parts: int) -> np.ndarray:
    """[parts][N][d] bf16 bits whose float sum approximates ``hidden``."""
    u = rng.standard_normal((parts,) + hidden.shape, dtype=np.float32)
    u *= np.float32(0.5)
    u -= u.mean(axis=0, dtype=np.float32, keepdims=True)
    u += hidden[None] / np.float32(parts)
    return to_bf16_bits(u)


def default_expert_cluster(E: int, G: int) -> np.ndarray:
    """Equal, contiguous expert placement: expert e lives in cluster e // (E/G)."""
    if E % G:
        raise ValueError("E must be a multiple of G for equal placement")
    return (np.arange(E) // (E // G)).astype(np.uint8)


def foe_row_cluster(N: int, H: int, G: int) -> np.ndarray:
    """Cluster holding FoE group h's copy of token i, flattened as [i*H + h].

    With G >= H each group owns G/H clusters and token i of group h sits on
    cluster h*(G/H) + (i mod G/H); with G < H group h sits on floor(h*G/H).
    """
    i = np.arange(N)[:, None]
    h = np.arange(H)[None, :]
    if G >= H:
        if G % H:
            raise ValueError("G must be a multiple of H when G >= H")
        c = h * (G // H) + (i % (G // H))
    else:
        c = (h * G) // H + 0 * i
    return c.reshape(-1).astype(np.uint8)


def make_route_inputs(N, d, E, K, P, G, V, seed, *, lut_mode="random",
                      ngram=False, zipf_s=1.1, noise=0.3, sample=0):
    """Inputs of the predict -> SRS -> gate -> top-K -> permute -> combine pass.

    ``sample`` > 0 draws another batch of the same model: new token ids,
    noise and partial split (streams [seed, 0|2|3, sample]), the same per-id
    base rows and gate weights."""
    key = (lambda st: _rng(seed, st)) if sample == 0 else (lambda st: _rng(seed, st, sample))
    tok = zipf_ids(key(0), N, V, zipf_s)
    ids_present = np.unique(tok).astype(np.int32)
    base = _base_rows(seed, ids_present, d)
    where = np.searchsorted(ids_present, tok)
    hidden = key(2).standard_normal((N, d), dtype=np.float32)
    hidden *= np.float32(noise)
    hidden += base[where]
    partials = _zero_sum_split(key(3), hidden, P)
    del hidden
    w = to_bf16_bits(_rng(seed, 4).standard_normal((E, d), dtype=np.float32)
                     / np.float32(np.sqrt(d)))
    r5 = _rng(seed, 5)
    lut = r5.integers(0, G, V, dtype=np.uint8)
    conf = r5.integers(0, 256, V, dtype=np.uint8)
    out = dict(
        tok=tok, partials=partials, w=w, lut=lut,
        expert_cluster=default_expert_cluster(E, G),
        ids_present=ids_present, base_present=to_bf16_bits(base),
        N=N, d=d, E=E, K=K, P=P, G=G, V=V, lut_mode=lut_mode,
    )
    if ngram:
        out["conf"] = conf
        out["ngram"] = _rng(seed, 6).integers(0, G, (G, G), dtype=np.uint8)
        r7 = _rng(seed, 7)
        out["prev2"] = r7.integers(0, G, N, dtype=np.uint8)
        out["prev1"] = r7.integers(0, G, N, dtype=np.uint8)
    return out


def make_foe_inputs(N, d, E, H, K, G, V, seed, *, zipf_s=1.1, noise=0.3):
    """Inputs of the grouped (FoE) pass: H per-group activations [H][N][d]."""
    tok = zipf_ids(_rng(seed, 0), N, V, zipf_s)
    ids_present = np.unique(tok).astype(np.int32)
    base = _base_rows(seed, ids_present, d)
    where = np.searchsorted(ids_present, tok)
    hidden = _rng(seed, 2).standard_normal((N, d), dtype=np.float32)
    hidden *= np.float32(noise)
    hidden += base[where]
    x = _zero_sum_split(_rng(seed, 3), hidden, H)
    del hidden
    w = to_bf16_bits(_rng(seed, 4).standard_normal((E, d), dtype=np.float32)
                     / np.float32(np.sqrt(d)))
    return dict(tok=tok, x=x, w=w, expert_cluster=default_expert_cluster(E, G),
                row_cluster=foe_row_cluster(N, H, G),
                N=N, d=d, E=E, H=H, K=K, G=G, V=V)


def make_predictor_layer(cfg: PredictorConfig, l: int, N=None, sample=0):
    """Inputs for source layer l (0 <= l < L-1) of the q_l predictor workload.

    r_l ~ N(0, 1) bf16; d_l ~ N(0, dvec_var) float32; the next layer's gate
    W_{l+1} ~ N(0, 1/d) bf16; the next layer's true router input
    s_{l+1} = bf16(r_l + drift * N(0, 1)); on estimator layers a 2-layer MLP
    d -> hd -> E with W ~ N(0, 1/fan_in) bf16 and biases ~ N(0, 0.01).
    """
    if not 0 <= l < cfg.L - 1:
        raise ValueError("source layer out of range")
    N = cfg.N if N is None else N
    d, E, hd = cfg.d, cfg.E, cfg.hd
    # sample > 0: another batch of the same model (new r_l and drift noise)
    key = (lambda st: _rng(cfg.seed, st, l)) if sample == 0 else \
        (lambda st: _rng(cfg.seed, st, l, sample))
    r = to_bf16_bits(key(10).standard_normal((N, d), dtype=np.float32))
    dvec = (_rng(cfg.seed, 11, l).standard_normal(d, dtype=np.float32)
            * np.float32(np.sqrt(cfg.dvec_var)))
    w_next = to_bf16_bits(_rng(cfg.seed, 12, l + 1).standard_normal((E, d), dtype=np.float32)
                          / np.float32(np.sqrt(d)))
    s = from_bf16_bits(r) + np.float32(cfg.drift) * key(13).standard_normal(
        (N, d), dtype=np.float32)
    out = dict(r=r, dvec=dvec, w_next=w_next, s_next=to_bf16_bits(s),
               N=N, d=d, E=E, K=cfg.K, hd=hd, eps=cfg.eps, estimator=l in cfg.est_layers)
    if l in cfg.est_layers:
        g = _rng(cfg.seed, 14, l)
        out["w1"] = to_bf16_bits(g.standard_normal((hd, d), dtype=np.float32) / np.float32(np.sqrt(d)))
        out["b1"] = g.standard_normal(hd, dtype=np.float32) * np.float32(0.1)
        out["w2"] = to_bf16_bits(g.standard_normal((E, hd), dtype=np.float32) / np.float32(np.sqrt(hd)))
        out["b2"] = g.standard_normal(E, dtype=np.float32) * np.float32(0.1)
    return out


def first_tokens(inp: dict, n: int) -> dict:
    """The first n tokens of a drawn batch (route, FoE or predictor layer):
    every per-token array cut to its first n tokens, every table and weight
    kept as it is. A batch drawn with N=n is not this one (the P-way split
    draws all N tokens of a part before the next part)."""
    N = inp["N"]
    n = min(n, N)
    out = dict(inp, N=n)
    for k in ("tok", "prev2", "prev1", "r", "s_next"):
        if k in inp:
            out[k] = inp[k][:n]
    for k in ("partials", "x"):
        if k in inp:
            out[k] = np.ascontiguousarray(inp[k][:, :n])
    if "row_cluster" in inp:
        out["row_cluster"] = inp["row_cluster"][: n * inp["H"]]
    return out


def make_config_inputs(name: str, N=None, sample=0):
    """Inputs of a named workload (route or FoE); N overrides the token count;
    ``sample`` > 0 draws another batch of a routing workload's model."""
    cfg = get_config(name)
    n = cfg.N if N is None else N
    if isinstance(cfg, RouteConfig):
        return make_route_inputs(n, cfg.d, cfg.E, cfg.K, cfg.P, cfg.G, cfg.V, cfg.seed,
                                 lut_mode=cfg.lut_mode, ngram=cfg.ngram,
                                 zipf_s=cfg.zipf_s, noise=cfg.noise, sample=sample)
    if isinstance(cfg, FoEConfig):
        return make_foe_inputs(n, cfg.d, cfg.E, cfg.H, cfg.K, cfg.G, cfg.V, cfg.seed,
                               zipf_s=cfg.zipf_s, noise=cfg.noise)
    raise ValueError(f"{name} is a per-layer workload; use make_predictor_layer")
