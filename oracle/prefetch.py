"""Plain definition of speculative expert prefetch on one GPU (oracle).

TEST INFRASTRUCTURE ONLY (see the package docstring).

"Speculating Experts Accelerates Inference for Mixture-of-Experts", technical
summary items 1 and 2 (and the analogy section before them): with the expert
weights offloaded to CPU memory, on-demand loading copies a layer's selected
experts to the GPU only after its router has run; prefetching instead
predicts the next layer's experts from q_l while the current layer computes,
copies them ahead, and speculative execution runs the prefetched experts
without waiting for the true router (item 2.B). Item 4 scores predictions by
hit rate.

The page describes single-request decoding, where the prefetched set is the
K predicted experts of one token. For a batch of n tokens and a staging
buffer of C expert slots the reading taken here is:

* plan: count how often each expert is named by the batch's predicted picks;
  the distinct predicted experts, ordered by count (descending, ties to the
  lower index), fill the C slots in order; unused slots hold -1;
* copy: slot i receives the weights of expert list[i] (a byte copy of that
  expert's block of the weight bank);
* coverage: a true pick (token, expert) is covered when its expert sits in a
  slot; the true experts that sit in no slot are the misses, the experts an
  on-demand load would still have to copy (listed in index order).

With n = 1 and C >= K the plan is the token's predicted set and coverage is
|pred ∩ true|, the hit count of item 4.
"""

from __future__ import annotations

import numpy as np


def prefetch_plan(pred, E, C):
    """(list int32[C], n_listed, counts int64[E]) from predicted picks pred[n][K].

    Picks outside [0, E) are ignored (the GPU flags them)."""
    counts = np.zeros(E, dtype=np.int64)
    for p in np.asarray(pred).ravel():
        if 0 <= p < E:
            counts[p] += 1
    named = [e for e in range(E) if counts[e] > 0]
    named.sort(key=lambda e: (-counts[e], e))
    chosen = named[:C]
    lst = np.full(C, -1, dtype=np.int32)
    lst[:len(chosen)] = chosen
    return lst, len(chosen), counts


def prefetch_copy(bank, lst, slots):
    """slots[i] = bank[lst[i]] for every slot with an expert in [0, E); the
    other slots keep their bytes. bank uint8[E][B], slots uint8[C][B]."""
    out = np.array(slots, copy=True)
    E = bank.shape[0]
    for i, e in enumerate(lst):
        if 0 <= e < E:
            out[i] = bank[e]
    return out


def prefetch_coverage(true, lst, E):
    """(covered picks, miss list int32[E] padded with -1, n_miss)."""
    inset = np.zeros(E, dtype=bool)
    for e in lst:
        if 0 <= e < E:
            inset[e] = True
    covered = 0
    present = np.zeros(E, dtype=bool)
    for t in np.asarray(true).ravel():
        if 0 <= t < E:
            present[t] = True
            covered += int(inset[t])
    missing = [e for e in range(E) if present[e] and not inset[e]]
    miss = np.full(E, -1, dtype=np.int32)
    miss[:len(missing)] = missing
    return covered, miss, len(missing)
