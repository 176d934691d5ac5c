"""Speculative expert prefetch on the GPU against the oracle ("Speculating
Experts Accelerates Inference for Mixture-of-Experts", items 1, 2 and 4):
the plan and the coverage bit for bit, the slot copy byte for byte from
pinned host memory (read by the kernel over PCIe) and from device memory, at
small sizes, at decode sizes with Qwen3-30B-A3B-sized experts, and under a
replayed graph."""


import numpy as np
import pytest
import torch

import token_routing_speculation_amd as tr
from oracle import prefetch as opf

from gpu_helpers import dev, host

pytestmark = pytest.mark.gpu

QWEN3_EXPERT_BYTES = 3 * 2048 * 768 * 2   # gate, up and down projections in bf16


def _picks(n, K, E, seed, skew=0.0):
    rng = np.random.default_rng(seed)
    p = 1.0 / np.arange(1, E + 1) ** skew
    p /= p.sum()
    return np.stack([rng.choice(E, K, replace=False, p=p) for _ in range(n)]).astype(np.int32) \
        if n else np.zeros((0, K), np.int32)


CASES = [(1, 8, 128, 8, 0.0), (1, 8, 128, 16, 0.0), (0, 8, 64, 8, 0.0), (37, 4, 16, 5, 1.0),
         (8192, 8, 128, 128, 1.0), (8192, 8, 128, 32, 0.5), (5000, 6, 160, 64, 1.2),
         (300, 2, 1024, 1024, 0.0), (3, 16, 1024, 40, 0.0), (64, 1, 2, 1, 0.0)]


@pytest.mark.parametrize("n,K,E,C,skew", CASES)
def test_plan_and_coverage(n, K, E, C, skew):
    pred = _picks(n, K, E, n + E + C, skew)
    truth = _picks(n, K, E, n + E + C + 1, skew)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    lst, nl = tr.prefetch_plan(dev(pred), E, C, err=err)
    wl, wnl, _ = opf.prefetch_plan(pred, E, C)
    assert np.array_equal(host(lst), wl) and host(nl)[0] == wnl
    cov = torch.zeros(1, dtype=torch.int64, device="cuda")
    miss, nm = tr.prefetch_coverage(dev(truth), lst, E, cov, err=err)
    wc, wm, wnm = opf.prefetch_coverage(truth, wl, E)
    assert host(cov)[0] == wc and np.array_equal(host(miss), wm) and host(nm)[0] == wnm
    tr.prefetch_coverage(dev(truth), lst, E, cov)          # the count accumulates
    assert host(cov)[0] == 2 * wc
    assert host(err)[0] == 0


def test_out_of_range_picks_are_flagged_and_skipped():
    pred = np.array([[3, 70, 1], [3, -2, 5]], np.int32)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    lst, nl = tr.prefetch_plan(dev(pred), 64, 8, err=err)
    wl, wnl, _ = opf.prefetch_plan(pred, 64, 8)
    assert np.array_equal(host(lst), wl) and host(nl)[0] == wnl == 3
    assert host(err)[0] & tr.EBIT_EXPERT_RANGE
    err.zero_()
    cov = torch.zeros(1, dtype=torch.int64, device="cuda")
    miss, nm = tr.prefetch_coverage(dev(pred), lst, 64, cov, err=err)
    wc, wm, wnm = opf.prefetch_coverage(pred, wl, 64)
    assert host(cov)[0] == wc and np.array_equal(host(miss), wm) and host(nm)[0] == wnm
    assert host(err)[0] & tr.EBIT_EXPERT_RANGE


def _pinned_bank(E, B, seed):
    bank = torch.empty((E, B), dtype=torch.uint8, pin_memory=True)
    g = torch.Generator().manual_seed(seed)
    bank.copy_(torch.randint(0, 256, (E, B), dtype=torch.uint8, generator=g))
    return bank


@pytest.mark.parametrize("E,B,C,where", [(16, 4096, 5, "host"), (16, 4096, 5, "device"),
                                         (128, 16, 128, "host"), (40, 65552, 7, "host"),
                                         (3, 1 << 20, 3, "device")])
def test_copy(E, B, C, where):
    bank = _pinned_bank(E, B, E + B)
    if where == "device":
        bank = bank.cuda()
    rng = np.random.default_rng(C)
    lst = rng.choice(E, C, replace=False).astype(np.int32)
    lst[C // 2] = -1                                   # an empty slot keeps its bytes
    slots0 = rng.integers(0, 256, (C, B), dtype=np.uint8)
    slots = dev(slots0)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    tr.prefetch_copy(bank, dev(lst), slots, err=err)
    want = opf.prefetch_copy(bank.cpu().numpy(), lst, slots0)
    assert np.array_equal(host(slots), want)
    assert host(err)[0] == 0


@pytest.mark.parametrize("lst,where", [([3, 4, 5, -1, 9, 10], "host"), ([7, 0, 1, 2, -1, -1], "host"),
                                       ([11, 10, 9, 8, 7, 6], "device"), ([-1] * 6, "host")])
def test_issue_dma(lst, where):
    E, B = 12, 12288
    bank = _pinned_bank(E, B, 77)
    if where == "device":
        bank = bank.cuda()
    slots0 = np.random.default_rng(1).integers(0, 256, (len(lst), B), dtype=np.uint8)
    slots = dev(slots0)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    tr.prefetch_issue(bank, torch.tensor(lst, dtype=torch.int32), slots, stream=s)
    s.synchronize()
    want = opf.prefetch_copy(bank.cpu().numpy(), np.array(lst), slots0)
    assert np.array_equal(host(slots), want)


def test_issue_from_a_plan_copied_back():
    """The plan runs on the GPU; its list comes back to pinned host memory;
    the DMA copies run on a second stream and the compute stream waits."""
    E, C = 12, 8
    bank = _pinned_bank(E, QWEN3_EXPERT_BYTES, 6)
    pred = _picks(1, 8, E, 10)
    lst, nl = tr.prefetch_plan(dev(pred), E, C)
    lst_h = torch.empty(C, dtype=torch.int32, pin_memory=True)
    lst_h.copy_(lst, non_blocking=True)
    done = torch.cuda.Event()
    done.record()
    done.synchronize()
    slots = torch.zeros((C, QWEN3_EXPERT_BYTES), dtype=torch.uint8, device="cuda")
    cs = torch.cuda.Stream()
    cs.wait_stream(torch.cuda.current_stream())
    tr.prefetch_issue(bank, lst_h, slots, stream=cs)
    torch.cuda.current_stream().wait_stream(cs)
    wl, _, _ = opf.prefetch_plan(pred, E, C)
    assert np.array_equal(lst_h.numpy(), wl)
    want = opf.prefetch_copy(bank.numpy(), wl, np.zeros((C, QWEN3_EXPERT_BYTES), np.uint8))
    assert np.array_equal(host(slots), want)


def test_copy_qwen3_experts_from_pinned_memory():
    E, C = 12, 8
    bank = _pinned_bank(E, QWEN3_EXPERT_BYTES, 5)
    pred = _picks(1, 8, E, 9)
    lst, nl = tr.prefetch_plan(dev(pred), E, C)
    slots = torch.zeros((C, QWEN3_EXPERT_BYTES), dtype=torch.uint8, device="cuda")
    tr.prefetch_copy(bank, lst, slots)
    wl, _, _ = opf.prefetch_plan(pred, E, C)
    want = opf.prefetch_copy(bank.numpy(), wl, np.zeros((C, QWEN3_EXPERT_BYTES), np.uint8))
    assert np.array_equal(host(slots), want)


def test_copy_flags_a_list_entry_past_the_bank():
    bank = _pinned_bank(4, 64, 1)
    slots0 = np.full((2, 64), 7, np.uint8)
    slots = dev(slots0)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    tr.prefetch_copy(bank, dev(np.array([9, 2], np.int32)), slots, err=err)
    assert host(err)[0] & tr.EBIT_EXPERT_RANGE
    got = host(slots)
    assert np.array_equal(got[0], slots0[0]) and np.array_equal(got[1], bank[2].numpy())


def test_copy_refuses_pageable_host_memory():
    B = 256
    page = np.zeros(4 * B + 16, np.uint8)
    base = page.ctypes.data
    ptr = base + (-base) % 16                          # 16-byte aligned pageable address
    lst = dev(np.array([0, 1], np.int32))
    slots = torch.zeros((2, B), dtype=torch.uint8, device="cuda")
    st = tr.lib().prefetch_copy(ptr, 4, B, lst.data_ptr(), 2, slots.data_ptr(), None,
                                torch.cuda.current_stream().cuda_stream)
    assert st == 7                                     # ROUTE_ERR_NOT_MAPPED
    hl = np.array([0, 1], np.int32)
    st = tr.lib().prefetch_issue(ptr, 4, B, hl.ctypes.data, 2, slots.data_ptr(),
                                 torch.cuda.current_stream().cuda_stream)
    assert st == 7
    with pytest.raises(ValueError):
        tr.prefetch_copy(torch.zeros((4, B), dtype=torch.uint8), lst, slots)
    with pytest.raises(ValueError):
        tr.prefetch_issue(torch.zeros((4, B), dtype=torch.uint8), torch.tensor([0, 1],
                          dtype=torch.int32), slots)
    assert (host(slots) == 0).all()


def test_graph_replay_matches_eager():
    """plan -> copy -> coverage captured once and replayed with new picks."""
    E, B, C, K = 32, 2048, 8, 4
    bank = _pinned_bank(E, B, 2)
    pred_d = torch.zeros((3, K), dtype=torch.int32, device="cuda")
    true_d = torch.zeros((3, K), dtype=torch.int32, device="cuda")
    lst = torch.empty(C, dtype=torch.int32, device="cuda")
    nl = torch.empty(1, dtype=torch.int32, device="cuda")
    slots = torch.zeros((C, B), dtype=torch.uint8, device="cuda")
    cov = torch.zeros(1, dtype=torch.int64, device="cuda")
    miss = torch.empty(E, dtype=torch.int32, device="cuda")
    nm = torch.empty(1, dtype=torch.int32, device="cuda")

    def body():
        tr.prefetch_plan(pred_d, E, C, lst=lst, nlist=nl)
        tr.prefetch_copy(bank, lst, slots)
        tr.prefetch_coverage(true_d, lst, E, cov, miss=miss, nmiss=nm)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        body()
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        body()
    torch.cuda.synchronize()
    cov.zero_()                                        # the warm-up call counted too
    total = 0
    for rep in range(4):
        pred = _picks(3, K, E, 100 + rep, 1.0)
        truth = _picks(3, K, E, 200 + rep, 1.0)
        pred_d.copy_(torch.from_numpy(pred))
        true_d.copy_(torch.from_numpy(truth))
        g.replay()
        torch.cuda.synchronize()
        wl, wnl, _ = opf.prefetch_plan(pred, E, C)
        wc, wm, wnm = opf.prefetch_coverage(truth, wl, E)
        total += wc
        assert np.array_equal(host(lst), wl) and host(nl)[0] == wnl, rep
        assert host(cov)[0] == total and np.array_equal(host(miss), wm) and host(nm)[0] == wnm
        got = host(slots)
        for i, e in enumerate(wl):
            if e >= 0:
                assert np.array_equal(got[i], bank[e].numpy()), (rep, i)
        # eager work between replays
        tr.prefetch_plan(pred_d, E, C)
        torch.cuda.synchronize()
