"""moe_permute_noalloc (the dispatch on the library's static per-GPU scratch)
against moe_permute with a caller workspace, through the C ABI: every map
and every dispatched row bit for bit, on two calls in a row whose second is
smaller (the scratch keeps the first call's table), and against the oracle's
stable sort and gather."""
import numpy as np
import pytest
import torch

import oracle
import token_routing_speculation_amd as tr

from tests.gpu_helpers import dev, host

pytestmark = pytest.mark.gpu

# (n, E, K, H, d) pairs: the second call of each pair is the smaller one
PAIRS = [((16384, 160, 6, 1, 512), (1000, 8, 2, 1, 64)),
         ((32768, 64, 8, 4, 256), (4097, 64, 8, 4, 128)),
         ((20000, 1024, 16, 1, 64), (77, 3, 3, 1, 16)),
         ((4096, 8, 2, 1, 4096), (1, 4, 2, 2, 8))]


def _case(n, E, K, H, d, seed):
    rng = np.random.default_rng(seed)
    lg = rng.standard_normal((n, E)).astype(np.float32)
    idx, _ = tr.route_topk(dev(lg), K, H, 1)
    src = rng.integers(0, 1 << 16, (H, n, d), dtype=np.uint16)
    return idx, src


def _outputs(n, E, K, d):
    z = lambda shape, dt: torch.full(shape, -7, dtype=dt, device="cuda")
    return (z((E + 1,), torch.int32), z((n * K,), torch.int32), z((n * K,), torch.int32),
            z((n * K, d), torch.int16).view(torch.bfloat16))


@pytest.mark.parametrize("big,small", PAIRS)
def test_noalloc_matches_moe_permute_twice(big, small):
    for call, (n, E, K, H, d) in enumerate((big, small)):
        idx, src = _case(n, E, K, H, d, seed=n + E + call)
        srcd = dev(src)
        err = torch.zeros(1, dtype=torch.int32, device="cuda")
        a = _outputs(n, E, K, d)
        tr.moe_permute_noalloc(idx, E, srcd, H, *a, err=err)
        b = tr.moe_permute(idx, E, srcd, H)
        torch.cuda.synchronize()
        assert int(err.item()) == 0
        for x, y in zip(a, b):
            assert np.array_equal(host(x), host(y))
        want = oracle.moe_permute(host(idx), E, H, src)
        assert np.array_equal(host(a[0]), want["expert_offsets"])
        assert np.array_equal(host(a[1]), want["slot_of_pair"])
        assert np.array_equal(host(a[2]), want["pair_of_slot"])
        assert np.array_equal(host(a[3]), want["disp"])


def test_noalloc_indices_only_and_empty():
    idx = dev(np.array([[3, 1], [1, 0], [3, 2]], dtype=np.int32))
    offs, sop, pos, disp = tr.moe_permute_noalloc(idx, 4)
    assert disp is None
    assert host(offs).tolist() == [0, 1, 3, 4, 6]
    assert host(pos).tolist() == [3, 1, 2, 5, 0, 4]
    empty = torch.empty((0, 2), dtype=torch.int32, device="cuda")
    offs, *_ = tr.moe_permute_noalloc(empty, 5)
    assert host(offs).tolist() == [0] * 6


def test_noalloc_flags_bad_expert():
    idx = dev(np.array([[0, 9], [1, 2]], dtype=np.int32))
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    tr.moe_permute_noalloc(idx, 4, err=err)
    torch.cuda.synchronize()
    assert int(err.item()) & tr.EBIT_EXPERT_RANGE
