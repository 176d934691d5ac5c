"""GPU parity of srs_shuffle_gate (the shuffled reduce and the router product
on its output, one kernel): every srs_shuffle output bit-exact against the
oracle's shuffle, the logits against the oracle's gate on the oracle's
reduced rows (the gate's tolerances), and the two-call GPU path on the same
inputs (the same bytes for every shuffle output; logits up to the order of the
binary32 sums)."""
import numpy as np
import pytest
import torch

import oracle
import token_routing_speculation_amd as tr
from synth import to_bf16_bits
from tests.gpu_helpers import dev, host, assert_rel, sync

pytestmark = pytest.mark.gpu

LOGIT_TOL = 1e-2      # the gate's stated bar (max relative error, row-rms floored)
F32_TOL = 1e-4        # binary32 accumulation of exact bf16 products
PAIR_TOL = 1e-5       # against route_gate on the same rows: only the sum order differs


def _bf16(shape, seed, scale=1.0):
    return to_bf16_bits((np.random.default_rng(seed).standard_normal(shape) * scale).astype(np.float32))


# (n, d, P, G, E): one row, less than a tile, exactly one tile at the
# shortest K (two steps), several tiles with a ragged tail, every supported
# P, E from 1 to 160, the maximum cluster count, the DeepSeek-V2 row length
CASES = [(1, 128, 1, 2, 160), (63, 256, 2, 3, 160), (64, 128, 2, 8, 160),
         (1000, 512, 2, 8, 160), (777, 384, 4, 5, 150), (513, 1024, 1, 8, 33),
         (300, 640, 2, 256, 1), (129, 256, 4, 7, 129), (2049, 5120, 2, 8, 160),
         (4133, 2048, 2, 16, 64)]


def _inputs(n, d, P, G, E):
    parts = _bf16((P, n, d), n * 7 + d + P)
    dest = np.random.default_rng(n + G).integers(0, G, n, dtype=np.uint8) if G < 256 else \
        np.random.default_rng(n).integers(0, 256, n, dtype=np.uint8)
    w = _bf16((E, d), E + d, 1 / np.sqrt(d))
    return parts, dest, w


@pytest.mark.parametrize("n,d,P,G,E", CASES)
def test_srs_gate_against_oracle(n, d, P, G, E):
    parts, dest, w = _inputs(n, d, P, G, E)
    want = oracle.srs_shuffle(parts, dest.astype(np.int64), G)
    out, offs, ros, sor, rc, logits = tr.srs_shuffle_gate(dev(parts), dev(dest), G, dev(w))
    assert np.array_equal(host(offs), want["offsets"])
    assert np.array_equal(host(ros), want["row_of_src"])
    assert np.array_equal(host(sor), want["src_of_row"])
    assert np.array_equal(host(rc), want["row_cluster"])
    assert np.array_equal(host(out), want["out"])
    ref = oracle.route_gate(want["out"], w)
    got = host(logits)
    assert_rel(got, ref, LOGIT_TOL, "fused logits")
    assert_rel(got, ref, F32_TOL, "fused logits (binary32 level)")


@pytest.mark.parametrize("n,d,P,G,E", [(1000, 512, 2, 8, 160), (777, 384, 4, 5, 150),
                                       (2049, 5120, 2, 8, 160)])
def test_srs_gate_equals_two_calls(n, d, P, G, E):
    parts, dest, w = _inputs(n, d, P, G, E)
    pd, dd, wd = dev(parts), dev(dest), dev(w)
    o1, f1, r1, s1, c1 = tr.srs_shuffle(pd, dd, G)
    l1 = tr.route_gate(o1, wd)
    o2, f2, r2, s2, c2, l2 = tr.srs_shuffle_gate(pd, dd, G, wd)
    for a, b in ((o1, o2), (f1, f2), (r1, r2), (s1, s2), (c1, c2)):
        assert torch.equal(a, b)
    assert_rel(host(l2), host(l1), PAIR_TOL, "fused vs two calls")


@pytest.mark.parametrize("n,d,P", [(1, 128, 4), (333, 256, 2), (70, 4096, 1)])
def test_srs_gate_pure_reduce_without_dest(n, d, P):
    """One cluster, no sort: the kernel writes the offsets {0, n} and the
    identity maps itself (the buffers start out holding other values)."""
    parts = _bf16((P, n, d), 3 + n)
    w = _bf16((160, d), d, 1 / np.sqrt(d))
    want = oracle.srs_shuffle(parts, None, 1)
    fill = lambda k, dt: torch.full((k,), 7, dtype=dt, device="cuda")
    out, offs, ros, sor, rc, logits = tr.srs_shuffle_gate(
        dev(parts), None, 1, dev(w), offsets=fill(2, torch.int32), row_of_src=fill(n, torch.int32),
        src_of_row=fill(n, torch.int32), row_cluster=fill(n, torch.uint8))
    assert np.array_equal(host(out), want["out"])
    assert host(offs).tolist() == [0, n]
    assert np.array_equal(host(ros), np.arange(n)) and np.array_equal(host(sor), np.arange(n))
    assert np.array_equal(host(rc), np.zeros(n))
    assert_rel(host(logits), oracle.route_gate(want["out"], w), F32_TOL, "pure-reduce logits")


def test_srs_gate_empty():
    parts = torch.empty((2, 0, 128), dtype=torch.bfloat16, device="cuda")
    dest = torch.empty((0,), dtype=torch.uint8, device="cuda")
    w = dev(_bf16((160, 128), 0))
    _, offs, *_, logits = tr.srs_shuffle_gate(parts, dest, 4, w)
    assert host(offs).tolist() == [0] * 5 and logits.shape == (0, 160)


def test_srs_gate_signed_zero_rows():
    """Partials of -0.0 sum to -0.0 (the binary32 fold from partial 0), and
    their logits are zero."""
    parts = np.full((2, 100, 128), 0x8000, dtype=np.uint16)
    dest = np.full(100, 3, dtype=np.uint8)
    w = _bf16((160, 128), 9)
    want = oracle.srs_shuffle(parts, dest, 4)
    out, offs, *_, logits = tr.srs_shuffle_gate(dev(parts), dev(dest), 4, dev(w))
    assert np.array_equal(host(out), want["out"]) and host(offs).tolist() == [0, 0, 0, 0, 100]
    assert np.all(host(logits) == 0.0)


def test_srs_gate_flags_bad_cluster_and_skips_its_row():
    """A key past G is flagged; its row gets neither a reduced row nor
    logits, and every other row is exact."""
    n, d, G, E = 200, 256, 4, 160
    parts = _bf16((2, n, d), 11)
    dest = np.random.default_rng(5).integers(0, G, n, dtype=np.uint8)
    dest[7] = 9
    w = _bf16((E, d), 12, 1 / np.sqrt(d))
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = torch.full((n, d), 3.0, dtype=torch.bfloat16, device="cuda")
    logits = torch.full((n, E), 5.0, dtype=torch.float32, device="cuda")
    _, offs, ros, sor, *_ = tr.srs_shuffle_gate(dev(parts), dev(dest), G, dev(w), out=out,
                                                logits=logits, err=err)
    sync()
    assert int(err.item()) & tr.EBIT_DEST_RANGE
    r = host(ros)
    assert r[7] == -1 and host(offs)[-1] == n - 1
    # the reduced rows of the others, each at its sorted row
    red = oracle.srs_shuffle(parts, np.zeros(n, dtype=np.int64), 1)["out"]
    o, lg = host(out), host(logits)
    ref = oracle.route_gate(red, w)
    keep = [i for i in range(n) if i != 7]
    assert np.array_equal(o[r[keep]], red[keep])
    assert_rel(lg[r[keep]], ref[keep], F32_TOL, "logits of the valid rows")
    # the one row no source maps to is left as it was
    free = sorted(set(range(n)) - set(r[keep].tolist()))
    assert len(free) == 1
    assert np.all(lg[free[0]] == 5.0)


def test_srs_gate_full_deepseek_shape_sampled():
    """The DeepSeek-V2-shaped launch (16384 x 5120, P = 2, G = 8, E = 160):
    every shuffle output equals the two-call path's bytes, and the logits of
    sampled rows match the oracle's gate on those rows."""
    n, d, P, G, E = 16384, 5120, 2, 8, 160
    g = torch.Generator(device="cuda").manual_seed(1)
    parts = torch.randn((P, n, d), device="cuda", generator=g).to(torch.bfloat16)
    dest = torch.randint(0, G, (n,), device="cuda", generator=g).to(torch.uint8)
    w = (torch.randn((E, d), device="cuda", generator=g) / d ** 0.5).to(torch.bfloat16)
    o1, f1, r1, s1, c1 = tr.srs_shuffle(parts, dest, G)
    o2, f2, r2, s2, c2, l2 = tr.srs_shuffle_gate(parts, dest, G, w)
    for a, b in ((o1, o2), (f1, f2), (r1, r2), (s1, s2), (c1, c2)):
        assert torch.equal(a, b)
    rows = np.random.default_rng(0).choice(n, 64, replace=False)
    rows = np.concatenate([rows, [0, n - 1]])
    x = host(o2)[rows]
    assert_rel(host(l2)[rows], oracle.route_gate(x, host(w)), F32_TOL, "sampled logits")
