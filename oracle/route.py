"""Plain definitions of every step of the routing/dispatch path (oracle).

TEST INFRASTRUCTURE ONLY (see the package docstring). bf16 tensors are
``uint16`` bit patterns. Index outputs are int64 numpy arrays; float outputs
are float64 unless the function says otherwise.
"""

from __future__ import annotations

import numpy as np
from scipy.special import erf

from .bf16 import bf16_to_f64, round_bf16


def _check(cond, msg):
    if not cond:
        raise ValueError(msg)


# --------------------------------------------------------------------------
# a1: route prediction from lookup tables
# --------------------------------------------------------------------------

def route_predict(tok, lut, conf=None, prev2=None, prev1=None, ngram=None,
                  conf_thr=128, G=None):
    """Predicted destination cluster of each token.

    "Speculative MoE" notes, section 4.1 (route-path prediction): the
    intra-layer model maps a token id to its most likely cluster through a
    profiled token table; the inter-layer model is a 2-gram Markov table over
    the cluster sequence of the preceding layers. The table with the higher
    confidence wins. The token table carries a confidence byte q (q/255); the
    2-gram table carries none, so the token table wins unless q < conf_thr,
    in which case the 2-gram table A[prev2][prev1] (the token's clusters at
    the two preceding layers) gives the prediction.
    """
    tok = np.asarray(tok)
    lut = np.asarray(lut, dtype=np.uint8)
    _check(tok.ndim == 1, "tok must be 1-D")
    _check(np.all((tok >= 0) & (tok < len(lut))), "token id out of vocabulary")
    dest = lut[tok].astype(np.int64)
    if conf is not None:
        _check(prev2 is not None and prev1 is not None and ngram is not None,
               "the 2-gram fallback needs prev2, prev1 and the table")
        ngram = np.asarray(ngram, dtype=np.uint8)
        g = ngram.shape[0]
        _check(ngram.shape == (g, g), "2-gram table must be square")
        prev2 = np.asarray(prev2).astype(np.int64)
        prev1 = np.asarray(prev1).astype(np.int64)
        fb = np.asarray(conf, dtype=np.uint8)[tok].astype(np.int64) < conf_thr
        _check(np.all((prev2[fb] < g) & (prev1[fb] < g)), "previous cluster out of range")
        dest[fb] = ngram[prev2[fb], prev1[fb]]
    if G is not None:
        _check(np.all(dest < G), "predicted cluster out of range")
    return dest


# --------------------------------------------------------------------------
# a2: shuffled reduce-scatter (SRS) on one GPU
# --------------------------------------------------------------------------

def srs_shuffle(partials, dest, G):
    """Reduce P partial activations, then move the rows into G cluster ranges.

    "Speculative MoE" notes, section 3.1 (s-TS): the tensor-parallel
    all-reduce is replaced by a reduce-scatter fused with a token shuffle, so
    each token's reduced activation lands with the cluster predicted for it.
    On one device the G destinations are G contiguous row ranges of one
    buffer, in cluster order, and tokens keep their original order inside a
    range (a stable sort by predicted cluster).

    The sum is the output's quantised code, so it follows the kernel's
    precision: binary32, a left fold p_0 + p_1 + ... + p_{P-1} (so a sum of
    negative zeros stays -0.0), rounded once to bf16 (nearest even).
    """
    partials = np.asarray(partials, dtype=np.uint16)
    _check(partials.ndim == 3, "partials must be [P][N][d]")
    P, N, d = partials.shape
    acc = bf16_to_f64(partials[0]).astype(np.float32)
    for p in range(1, P):
        acc = acc + bf16_to_f64(partials[p]).astype(np.float32)
    x = round_bf16(acc.astype(np.float64))
    if dest is None:
        _check(G == 1, "dest may be omitted only for a single cluster")
        dest = np.zeros(N, dtype=np.int64)
    dest = np.asarray(dest).astype(np.int64)
    _check(dest.shape == (N,), "dest must be [N]")
    _check(np.all((dest >= 0) & (dest < G)), "dest out of range")
    order = np.argsort(dest, kind="stable")
    row_of_src = np.empty(N, dtype=np.int64)
    row_of_src[order] = np.arange(N)
    counts = np.bincount(dest, minlength=G)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    return dict(out=x[order], offsets=offsets, row_of_src=row_of_src,
                src_of_row=order.astype(np.int64), row_cluster=dest[order],
                reduced=x)


# --------------------------------------------------------------------------
# a3: gate projection
# --------------------------------------------------------------------------

def route_gate(x, w):
    """Router logits g[i] = x_i . W^T over all E experts, in float64.

    "Federation of Experts (FoE)" article, per-layer comparison: the router
    scores g[i] of token i feed the (grouped) top-k. bf16 operands are
    decoded exactly; products and sums are float64.
    """
    x = bf16_to_f64(x)
    w = bf16_to_f64(w)
    _check(x.ndim == 2 and w.ndim == 2 and x.shape[1] == w.shape[1], "shape mismatch")
    return x @ w.T


# --------------------------------------------------------------------------
# a4: softmax + top-K, grouped top-k/H
# --------------------------------------------------------------------------

def route_topk(logits, K, H=1, renorm=1):
    """Top-K experts per token and their gate weights.

    "Federation of Experts (FoE)" article, grouped MoE block: group h owns
    experts E_h = [h*E/H, (h+1)*E/H) and picks its own top k/H by the router
    scores; H = 1 is plain top-K ("Speculative MoE" notes, section 1).

    Ranking is on the logits themselves under a total order: larger value
    first, the lower expert index first among equal values; -0.0 equals +0.0.
    Output slots are group-major and descending inside a group.

    Weights: renorm=1 gives the softmax over each group's selected logits
    (each group's weights sum to 1; H = 1 is the softmax over the K chosen);
    renorm=0 gives the full softmax over all E experts, read at the chosen
    ones.
    """
    v = np.asarray(logits, dtype=np.float64).copy()
    _check(v.ndim == 2, "logits must be [N][E]")
    N, E = v.shape
    _check(H >= 1 and E % H == 0 and K % H == 0, "E and K must be multiples of H")
    eg, kg = E // H, K // H
    _check(1 <= kg <= eg, "need 1 <= K/H <= E/H")
    v[v == 0.0] = 0.0  # fold -0.0 onto +0.0
    idx = np.empty((N, K), dtype=np.int64)
    for h in range(H):
        block = v[:, h * eg:(h + 1) * eg]
        order = np.argsort(-block, axis=1, kind="stable")[:, :kg]
        idx[:, h * kg:(h + 1) * kg] = order + h * eg
    sel = np.take_along_axis(v, idx, axis=1)
    w = np.empty((N, K), dtype=np.float64)
    if renorm:
        for h in range(H):
            s = sel[:, h * kg:(h + 1) * kg]
            e = np.exp(s - s.max(axis=1, keepdims=True))
            w[:, h * kg:(h + 1) * kg] = e / e.sum(axis=1, keepdims=True)
    else:
        m = v.max(axis=1, keepdims=True)
        z = np.exp(v - m).sum(axis=1, keepdims=True)
        w = np.exp(sel - m) / z
    return idx, w


# --------------------------------------------------------------------------
# a5: local activation rate counter
# --------------------------------------------------------------------------

def lar_count(idx, K, H, row_cluster, expert_cluster):
    """Number of (token, expert) activations that stay on the token's cluster.

    "Speculative MoE" notes, section 7 (local activation rate alpha: the
    share of activations routed to an expert on the token's own device);
    "Federation of Experts (FoE)" article (rho, the share resolved locally).
    Token i's copy for group h sits on row_cluster[i*H + h]; slot k of token
    i belongs to group k // (K/H). The rate is this count over N*K.
    """
    idx = np.asarray(idx).astype(np.int64)
    N = idx.shape[0]
    _check(idx.shape == (N, K) and K % H == 0, "idx must be [N][K]")
    rc = np.asarray(row_cluster).astype(np.int64).reshape(N, H)
    ec = np.asarray(expert_cluster).astype(np.int64)
    _check(np.all((idx >= 0) & (idx < len(ec))), "expert index out of range")
    group_of_slot = np.arange(K) // (K // H)
    return int(np.count_nonzero(ec[idx] == rc[:, group_of_slot]))


# --------------------------------------------------------------------------
# a6: expert-contiguous dispatch permutation
# --------------------------------------------------------------------------

def moe_permute(idx, E, H=1, src=None):
    """Dispatch: lay the (token, expert) pairs out expert by expert.

    "Speculative MoE" notes, section 1: dispatch sends each token's activation
    to every one of its K experts. On one device that is a stable sort of the
    pairs p = i*K + k by expert idx[i, k]; the pair's row is copied to its
    slot. With H groups the row for pair (i, k) is the group-(k // (K/H))
    activation of token i ("Federation of Experts (FoE)" article: experts of
    group h read r[h, i]).
    """
    idx = np.asarray(idx).astype(np.int64)
    _check(idx.ndim == 2, "idx must be [N][K]")
    N, K = idx.shape
    _check(K % H == 0, "K must be a multiple of H")
    keys = idx.reshape(-1)
    _check(np.all((keys >= 0) & (keys < E)), "expert index out of range")
    pair_of_slot = np.argsort(keys, kind="stable")
    slot_of_pair = np.empty(N * K, dtype=np.int64)
    slot_of_pair[pair_of_slot] = np.arange(N * K)
    counts = np.bincount(keys, minlength=E)
    expert_offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    out = dict(expert_offsets=expert_offsets, slot_of_pair=slot_of_pair,
               pair_of_slot=pair_of_slot.astype(np.int64))
    if src is not None:
        src = np.asarray(src, dtype=np.uint16)
        _check(src.ndim == 3 and src.shape[0] == H and src.shape[1] == N, "src must be [H][N][d]")
        p = pair_of_slot
        out["disp"] = src[(p % K) // (K // H), p // K]
    return out


# --------------------------------------------------------------------------
# a7: weighted combine (with the SAG unshuffle)
# --------------------------------------------------------------------------

def moe_combine(y, w, slot_of_pair, out_row=None):
    """Combine: out[out_row[j]] = sum_k w[j, k] * y[slot_of_pair[j*K + k]].

    "Speculative MoE" notes, section 1 (combine returns the expert outputs to
    the token and sums them) and section 3.1 (SAG returns shuffled tokens to
    their original positions: the out_row scatter). In the FoE layout the K
    slots span all H groups, so the same sum is the cross-group sum
    ("Federation of Experts (FoE)" article). float64 accumulation.
    """
    y = bf16_to_f64(y)
    w = np.asarray(w, dtype=np.float64)
    N, K = w.shape
    sop = np.asarray(slot_of_pair).astype(np.int64).reshape(N, K)
    _check(np.all((sop >= 0) & (sop < y.shape[0])), "slot out of range")
    o = np.einsum("jk,jkd->jd", w, y[sop])
    if out_row is None:
        return o
    out_row = np.asarray(out_row).astype(np.int64)
    _check(np.array_equal(np.sort(out_row), np.arange(N)), "out_row must be a permutation")
    out = np.empty_like(o)
    out[out_row] = o
    return out


# --------------------------------------------------------------------------
# a8: quasi-hidden state
# --------------------------------------------------------------------------

def route_qhidden(r, dvec, gamma=None, beta=None, eps=1e-5):
    """q_l = LN_{l+1}(d_l + r_l), LayerNorm over the hidden dimension.

    "Speculating Experts Accelerates Inference for Mixture-of-Experts",
    technical summary item 2.A: the default vector d_l plus the current
    residual r_l, normalised by the next layer's norm, approximates the next
    router input. Biased variance; gamma = 1 and beta = 0 when omitted.
    """
    v = bf16_to_f64(r) + np.asarray(dvec, dtype=np.float64)[None, :]
    mu = v.mean(axis=1, keepdims=True)
    var = ((v - mu) ** 2).mean(axis=1, keepdims=True)
    q = (v - mu) / np.sqrt(var + eps)
    if gamma is not None:
        q = q * np.asarray(gamma, dtype=np.float64)[None, :]
    if beta is not None:
        q = q + np.asarray(beta, dtype=np.float64)[None, :]
    return q


# --------------------------------------------------------------------------
# a9: lightweight neural estimator
# --------------------------------------------------------------------------

def gelu_erf(x):
    """GELU(x) = x * Phi(x) = 0.5 x (1 + erf(x / sqrt 2))."""
    x = np.asarray(x, dtype=np.float64)
    return 0.5 * x * (1.0 + erf(x / np.sqrt(2.0)))


def route_estimator(q, w1, b1, w2, b2):
    """Next-layer router logits from q_l through a 2-layer MLP.

    "Speculating Experts Accelerates Inference for Mixture-of-Experts",
    technical summary item 2.C: a shallow network maps q_l straight to the
    next layer's router logits, used on the early, high-drift layers.
    logits = GELU(q W1^T + b1) W2^T + b2, float64 throughout.
    """
    q = bf16_to_f64(q)
    h = gelu_erf(q @ bf16_to_f64(w1).T + np.asarray(b1, dtype=np.float64)[None, :])
    return h @ bf16_to_f64(w2).T + np.asarray(b2, dtype=np.float64)[None, :]


# --------------------------------------------------------------------------
# a10: prefetch hit counter
# --------------------------------------------------------------------------

def hit_count(pred, truth):
    """sum_i |pred_i intersect truth_i| over tokens.

    "Speculating Experts Accelerates Inference for Mixture-of-Experts",
    technical summary item 4 (hit rate of the predicted experts); the rate is
    this count over N*K.
    """
    pred = np.asarray(pred)
    truth = np.asarray(truth)
    _check(pred.shape == truth.shape and pred.ndim == 2, "pred and truth must be [N][K]")
    return int(sum(len(set(a.tolist()) & set(b.tolist())) for a, b in zip(pred, truth)))


# --------------------------------------------------------------------------
# offline table builder for the token -> cluster table
# --------------------------------------------------------------------------

def route_lut_build(ids, idx, w, expert_cluster, G, lut, conf=None):
    """Fill lut[ids[i]] (and conf) from each id's routing.

    "Speculative MoE" notes, section 4.1: the token-expert confidence table
    Pr(E_k | x) is reduced to a token -> cluster table. For id ids[i] with
    routing (idx[i], w[i]) the share of cluster c is the sum of the weights
    of the chosen experts placed on c; the table takes the cluster with the
    largest share (the lower cluster on ties) and the confidence byte
    round(255 * share), clamped to 255.

    The winner and the byte are integer codes decided by float arithmetic, so
    they follow the kernel's precision: binary32 shares accumulated over
    k = 0..K-1, then 255 * share and + 0.5 each rounded to binary32, then
    floor. ``lut``/``conf`` are modified in place and returned.
    """
    ids = np.asarray(ids).astype(np.int64)
    idx = np.asarray(idx).astype(np.int64)
    w32 = np.asarray(w, dtype=np.float32)
    ec = np.asarray(expert_cluster).astype(np.int64)
    n, K = idx.shape
    _check(len(ids) == n and len(np.unique(ids)) == n, "ids must be distinct, one per row")
    _check(np.all((ids >= 0) & (ids < len(lut))), "id out of vocabulary")
    for i in range(n):
        share = np.zeros(G, dtype=np.float32)
        for k in range(K):
            share[ec[idx[i, k]]] = np.float32(share[ec[idx[i, k]]] + w32[i, k])
        c = int(np.argmax(share))  # first maximum = lower cluster
        lut[ids[i]] = c
        if conf is not None:
            t = np.float32(np.float32(255.0) * share[c])
            t = np.float32(t + np.float32(0.5))
            conf[ids[i]] = int(min(255.0, max(0.0, np.floor(t))))
    return lut, conf
