"""Pins for the oracle's bf16 codec: hand-derived ties, PyTorch's CPU
conversion, and brute-force nearest-value search with exact rationals."""
import os
from fractions import Fraction

import numpy as np
import torch

from oracle.bf16 import bf16_to_f64, round_bf16, f32_to_bf16

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "bf16_rne.txt")


def _golden():
    rows = []
    for line in open(GOLDEN):
        line = line.split("#")[0].strip()
        if line:
            a, b = line.split()
            rows.append((int(a, 16), int(b, 16)))
    return rows


def test_hand_derived_cases():
    rows = _golden()
    assert len(rows) >= 15
    f = np.array([a for a, _ in rows], dtype=np.uint32).view(np.float32)
    got = f32_to_bf16(f)
    want = np.array([b for _, b in rows], dtype=np.uint16)
    assert np.array_equal(got, want), [(hex(a), hex(g), hex(w)) for (a, _), g, w in zip(rows, got, want) if g != w]


def test_matches_torch_on_random_binary32():
    rng = np.random.default_rng(7)
    bits = rng.integers(0, 2**32, 200000, dtype=np.uint64).astype(np.uint32)
    f = bits.view(np.float32)
    f = f[np.isfinite(f)]
    want = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(f32_to_bf16(f), want)


def test_matches_torch_on_exact_ties():
    rng = np.random.default_rng(8)
    hi = rng.integers(0, 0x7F7F, 50000, dtype=np.uint32)
    bits = (hi << 16) | 0x8000
    f = bits.view(np.float32)
    want = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(f32_to_bf16(f), want)


def _nearest_bf16_bruteforce(x: float) -> int:
    """Exact search over bf16 candidates around x, ties to even bit pattern."""
    base = int(np.float32(x).view(np.uint32) >> 16)
    cands = []
    for b in range(max(0, base - 3), base + 4):
        for s in (0, 0x8000):
            bb = (b & 0x7FFF) | s
            if (bb & 0x7F80) == 0x7F80:
                continue
            v = float(bf16_to_f64(np.array([bb], dtype=np.uint16))[0])
            cands.append((abs(Fraction(v) - Fraction(x)), bb & 1, bb))
    cands.sort()
    best = [c for c in cands if c[0] == cands[0][0]]
    even = [c for c in best if c[1] == 0]
    return (even or best)[0][2]


def test_float64_inputs_round_once_to_nearest():
    rng = np.random.default_rng(9)
    x = rng.standard_normal(3000) * np.exp2(rng.integers(-20, 20, 3000))
    # include values a hair off bf16 midpoints, which a double rounding via
    # binary32 would get wrong
    mid = bf16_to_f64(rng.integers(0x3000, 0x5000, 500, dtype=np.uint16)) * (1 + 2.0**-8)
    x = np.concatenate([x, mid * (1 + 2.0**-30), mid * (1 - 2.0**-30)])
    got = round_bf16(x)
    want = np.array([_nearest_bf16_bruteforce(float(v)) for v in x], dtype=np.uint16)
    assert np.array_equal(got, want)


def test_decode_is_exact():
    u = np.arange(0, 2**16, dtype=np.uint32).astype(np.uint16)
    d = bf16_to_f64(u)
    t = torch.from_numpy(u.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    fin = np.isfinite(t)
    assert np.array_equal(d[fin], t[fin])
    assert np.array_equal(np.isnan(d), np.isnan(t))
