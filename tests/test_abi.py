"""The C ABI: libroute.so loads, exports every entry point include/route.h
declares, and rejects host-checkable errors with the documented status
before anything is enqueued (these calls never reach a GPU)."""
import ctypes
import os
import re

import pytest

import token_routing_speculation_amd as tr

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "route.h")

OK, NULL, SHAPE, ALIGN, UNSUP, WS = 0, 1, 2, 3, 4, 5
A = 0x100000          # fake 16-byte aligned device address, never dereferenced
MIS = 0x100008        # 8-byte aligned only


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(tr.library_path()):
        from token_routing_speculation_amd.build import build
        build()
    return tr.lib()


def header_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return set(re.findall(r"^\s*(?:int|size_t|const char\*)\s+(\w+)\s*\(", src, flags=re.M))


def test_every_declared_symbol_is_exported(L):
    names = header_functions()
    assert len(names) == 49, names
    for n in names:
        assert hasattr(L, n), n
    assert names == set(tr.EXPORTS)


def test_status_strings(L):
    assert L.route_status_str(0) == b"ok"
    for s in range(1, 8):
        assert L.route_status_str(s) not in (b"ok", b"unknown status")
    assert L.route_status_str(99) == b"unknown status"


def test_gate_errors(L):
    f = L.route_gate
    assert f(None, 10, 64, A, 8, A, None) == NULL
    assert f(A, -1, 64, A, 8, A, None) == SHAPE
    assert f(A, 10, 60, A, 8, A, None) == SHAPE
    assert f(A, 10, 64, A, 1025, A, None) == UNSUP
    # rows longer than 4194304 with E > 32, on every kernel path (a multiple of 128 or not)
    assert f(A, 10, (1 << 22) + 128, A, 64, A, None) == UNSUP
    assert f(A, 10, (1 << 22) + 8, A, 160, A, None) == UNSUP
    assert f(MIS, 10, 64, A, 8, A, None) == ALIGN
    assert f(A, 0, 64, A, 8, A, None) == OK       # n = 0 is a no-op


def test_topk_errors(L):
    f = L.route_topk
    assert f(A, 10, 6, 4, 4, 1, A, None, None) == SHAPE      # E % H
    assert f(A, 10, 8, 3, 2, 1, A, None, None) == SHAPE      # K % H
    assert f(A, 10, 8, 10, 2, 1, A, None, None) == SHAPE     # K/H > E/H
    assert f(A, 10, 64, 17, 1, 1, A, None, None) == UNSUP
    assert f(A, 10, 2048, 4, 1, 1, A, None, None) == UNSUP
    assert f(None, 10, 8, 2, 1, 1, A, None, None) == NULL
    assert f(A, 0, 8, 2, 1, 1, A, None, None) == OK


def test_srs_errors(L):
    f = L.srs_shuffle
    ws = L.srs_shuffle_workspace_size(1000, 8)
    assert ws > 0
    args = lambda **k: dict(dict(partials=A, P=2, n=1000, d=64, dest=A, G=8, out=A, offs=A,
                                 ros=None, sor=None, rc=None, ws=A, wsb=ws, err=None, s=None), **k)
    call = lambda a: f(*a.values())
    assert call(args(wsb=ws - 1)) == WS
    assert call(args(ws=None)) == WS
    assert call(args(dest=None)) == NULL
    assert call(args(out=None)) == NULL
    assert call(args(d=12)) == SHAPE
    assert call(args(P=0)) == SHAPE
    assert call(args(P=17)) == UNSUP
    assert call(args(G=300)) == UNSUP
    assert call(args(partials=MIS)) == ALIGN



def test_srs_gate_errors(L):
    f = L.srs_shuffle_gate
    ws = L.srs_shuffle_workspace_size(1000, 8)
    args = lambda **k: dict(dict(partials=A, P=2, n=1000, d=256, dest=A, G=8, out=A, offs=A,
                                 ros=None, sor=None, rc=None, w=A, E=160, logits=A, ws=A, wsb=ws,
                                 err=None, s=None), **k)
    call = lambda a: f(*a.values())
    assert call(args(wsb=ws - 1)) == WS
    assert call(args(ws=None)) == WS
    assert call(args(dest=None)) == NULL
    assert call(args(w=None)) == NULL
    assert call(args(logits=None)) == NULL
    assert call(args(out=None)) == NULL
    assert call(args(offs=None)) == NULL
    assert call(args(d=12)) == SHAPE
    assert call(args(E=0)) == SHAPE
    assert call(args(n=-1)) == SHAPE
    # the fused kernel's shapes only: P in {1, 2, 4}, d % 128 == 0, E <= 160
    assert call(args(P=3)) == UNSUP
    assert call(args(P=8)) == UNSUP
    assert call(args(d=192)) == UNSUP
    assert call(args(d=64)) == UNSUP
    assert call(args(E=161)) == UNSUP
    assert call(args(G=300)) == UNSUP
    assert call(args(partials=MIS)) == ALIGN
    assert call(args(w=MIS)) == ALIGN

def test_srs_route_errors(L):
    f = L.srs_shuffle_route
    ws = L.srs_shuffle_workspace_size(1000, 8)
    args = lambda **k: dict(dict(partials=A, P=2, n=1000, d=512, dest=A, G=8, out=A, offs=A,
                                 ros=None, sor=None, rc=None, w=A, E=8, logits=A, K=2, renorm=1,
                                 idx=A, weights=A, ec=A, local=A, ws=A, wsb=ws, err=None,
                                 s=None), **k)
    call = lambda a: f(*a.values())
    assert call(args(wsb=ws - 1)) == WS
    assert call(args(ws=None)) == WS
    assert call(args(dest=None)) == NULL
    assert call(args(w=None)) == NULL
    assert call(args(idx=None)) == NULL
    assert call(args(out=None)) == NULL
    assert call(args(offs=None)) == NULL
    assert call(args(local=None)) == NULL      # the count needs both
    assert call(args(ec=None)) == NULL
    assert call(args(d=12)) == SHAPE
    assert call(args(E=0)) == SHAPE
    assert call(args(K=0)) == SHAPE
    assert call(args(K=9)) == SHAPE            # K > E
    assert call(args(n=-1)) == SHAPE
    # neither kernel: the lane-per-expert one needs E <= 64, the padded
    # router rows within 64 KiB of LDS, d <= 4096, P in {1, 2, 4} (four
    # partials up to d = 2048); the matrix-core one d % 128 == 0, E <= 160;
    # both K <= 16
    assert call(args(E=65, K=2, d=264)) == UNSUP
    assert call(args(E=161, d=4096)) == UNSUP
    assert call(args(E=40, d=520)) == UNSUP    # 41600 bytes, 81920 padded
    assert call(args(E=32, d=520, ws=None)) == WS   # 65536 padded: supported
    assert call(args(E=160, K=6, d=5120, ws=None)) == WS   # the matrix-core kernel
    assert call(args(E=1, K=1, d=4104)) == UNSUP
    assert call(args(P=3)) == UNSUP
    assert call(args(P=4, d=2056, E=4)) == UNSUP
    assert call(args(E=32, K=17, d=512)) == UNSUP
    assert call(args(G=300)) == UNSUP
    assert call(args(partials=MIS)) == ALIGN
    assert call(args(w=MIS)) == ALIGN
    assert call(args(out=MIS)) == ALIGN


def test_predict_sort_and_route_sorted_errors(L):
    f = L.route_predict_sort
    ws = L.route_predict_sort_workspace_size(1000, 8)
    args = lambda **k: dict(dict(tok=A, n=1000, lut=A, conf=None, vocab=5000, p2=None, p1=None,
                                 ng=None, G=8, thr=128, dest=A, offs=A, ros=A, sor=A, rc=None,
                                 ws=A, wsb=ws, err=None, s=None), **k)
    call = lambda a: f(*a.values())
    assert call(args(n=-1)) == SHAPE
    assert call(args(G=0)) == SHAPE
    assert call(args(vocab=0)) == SHAPE
    assert call(args(G=257)) == UNSUP
    assert call(args(offs=None)) == NULL
    assert call(args(ros=None)) == NULL
    assert call(args(sor=None)) == NULL
    assert call(args(dest=None)) == NULL
    assert call(args(conf=A)) == NULL          # the fallback needs prev2, prev1, ngram
    assert call(args(ws=None)) == WS
    assert call(args(wsb=ws - 1)) == WS
    assert L.route_predict_sort_workspace_size(1000, 300) == 0
    g = L.srs_route_sorted
    args = lambda **k: dict(dict(partials=A, P=2, n=1000, d=512, ros=A, dest=None, out=A, w=A,
                                 E=8, logits=None, K=2, renorm=1, idx=A, weights=None, ec=None,
                                 local=None, s=None), **k)
    call = lambda a: g(*a.values())
    assert call(args(K=9)) == SHAPE
    assert call(args(d=12)) == SHAPE
    assert call(args(E=161, d=4096)) == UNSUP
    assert call(args(K=17, E=32)) == UNSUP
    assert call(args(ros=None)) == NULL
    assert call(args(idx=None)) == NULL
    assert call(args(ec=A)) == NULL            # the count needs both
    assert call(args(out=MIS)) == ALIGN
    assert call(args(n=0, ros=None)) == OK


def test_predict_route_errors(L):
    f = L.srs_predict_route
    args = lambda **k: dict(dict(tok=A, n=1000, lut=A, conf=None, vocab=5000, p2=None, p1=None,
                                 ng=None, G=4, thr=128, partials=A, P=2, d=512, w=A, E=8, K=2,
                                 renorm=1, dest=A, offs=A, ros=A, sor=A, rc=None, out=A,
                                 logits=None, idx=A, weights=None, ec=None, local=None, err=None,
                                 s=None), **k)
    call = lambda a: f(*a.values())
    assert call(args(vocab=0)) == SHAPE
    assert call(args(G=0)) == SHAPE
    assert call(args(K=9)) == SHAPE
    assert call(args(d=12)) == SHAPE
    assert call(args(n=4097)) == UNSUP         # one row per wave of at most 256 workgroups
    assert call(args(G=17)) == UNSUP
    assert call(args(E=65)) == UNSUP            # the lane-per-expert kernel only
    assert call(args(P=3)) == UNSUP
    assert call(args(offs=None)) == NULL
    assert call(args(tok=None)) == NULL
    assert call(args(dest=None)) == NULL
    assert call(args(ros=None)) == NULL
    assert call(args(sor=None)) == NULL
    assert call(args(conf=A)) == NULL           # the fallback needs prev2, prev1, ngram
    assert call(args(idx=None)) == NULL
    assert call(args(ec=A)) == NULL             # the count needs both
    assert call(args(partials=MIS)) == ALIGN


def test_qest_hidden_errors(L):
    f = L.route_qest_hidden_packed
    args = lambda **k: dict(dict(r=A, dvec=A, g=None, b=None, n=100, d=2048, eps=1e-5, w1p=A,
                                 b1=A, hd=512, h=A, s=None), **k)
    call = lambda a: f(*a.values())
    assert call(args(d=12)) == SHAPE
    assert call(args(hd=0)) == SHAPE
    assert call(args(hd=12)) == SHAPE           # rows of whole 16-byte vectors
    assert call(args(eps=-1.0)) == SHAPE
    assert call(args(d=512)) == UNSUP          # q_l's tile sizes: 1024, 2048, 4096
    assert call(args(hd=1032)) == UNSUP
    assert call(args(b1=None)) == NULL
    assert call(args(w1p=None)) == NULL
    assert call(args(h=None)) == NULL
    assert call(args(r=MIS)) == ALIGN
    assert call(args(n=0)) == OK                # nothing to do


def test_qest_topk_errors(L):
    f = L.route_qest_topk_packed
    args = lambda **k: dict(dict(r=A, dvec=A, g=None, b=None, n=100, d=2048, eps=1e-5, w1p=A,
                                 b1=A, hd=512, w2p=A, b2=None, E=128, K=8, logits=None, idx=A,
                                 truth=None, hits=None, s=None), **k)
    call = lambda a: f(*a.values())
    assert call(args(d=12)) == SHAPE
    assert call(args(hd=12)) == SHAPE
    assert call(args(eps=-1.0)) == SHAPE
    assert call(args(K=0)) == SHAPE
    assert call(args(K=129)) == SHAPE          # K > E
    assert call(args(d=512)) == UNSUP          # q_l's tile sizes: 1024, 2048, 4096
    assert call(args(hd=768)) == UNSUP         # the hidden tile: 512 or 1024 wide
    assert call(args(E=257, K=8)) == UNSUP
    assert call(args(K=17)) == UNSUP
    assert call(args(b1=None)) == NULL
    assert call(args(w2p=None)) == NULL
    assert call(args(idx=None)) == NULL
    assert call(args(truth=A)) == NULL         # truth without hits
    assert call(args(w2p=MIS)) == ALIGN
    assert call(args(n=0)) == OK                # nothing to do


def test_predict_route_dispatch_errors(L):
    f = L.srs_predict_route_dispatch
    need = L.srs_predict_route_dispatch_workspace_size(1000, 4, 8)
    assert need == 256 + 4 * 8 * 256 * 4          # the count, then [G*E][256] int32
    assert L.srs_predict_route_dispatch_workspace_size(1000, 16, 32) == 0   # G*E > 256
    assert L.srs_predict_route_dispatch_workspace_size(4097, 4, 8) == 0
    args = lambda **k: dict(dict(tok=A, n=1000, lut=A, conf=None, vocab=5000, p2=None, p1=None,
                                 ng=None, G=4, thr=128, partials=A, P=2, d=512, w=A, E=8, K=2,
                                 renorm=1, dest=A, offs=A, ros=A, sor=A, rc=None, out=None,
                                 logits=None, idx=A, weights=A, ec=None, local=None, eoff=A,
                                 sop=A, pos=A, disp=A, ws=A, ws_bytes=need, err=None, s=None), **k)
    call = lambda a: f(*a.values())
    assert call(args(vocab=0)) == SHAPE
    assert call(args(K=9)) == SHAPE
    assert call(args(n=4097)) == UNSUP
    assert call(args(G=17)) == UNSUP
    assert call(args(E=65)) == UNSUP
    assert call(args(G=16, E=32)) == UNSUP      # more than 256 (cluster, expert) entries
    assert call(args(eoff=None)) == NULL
    assert call(args(offs=None)) == NULL
    assert call(args(weights=None)) == NULL     # the combine's weights are part of the dispatch
    assert call(args(sop=None)) == NULL
    assert call(args(pos=None)) == NULL
    assert call(args(disp=None)) == NULL
    assert call(args(ec=A)) == NULL
    assert call(args(disp=MIS)) == ALIGN
    assert call(args(out=MIS)) == ALIGN
    assert call(args(ws=None)) == WS
    assert call(args(ws_bytes=need - 1)) == WS
    assert call(args(ws=A + 16)) == WS          # 256-byte alignment


def test_route_grouped_errors(L):
    f = L.srs_route_grouped
    args = lambda **k: dict(dict(partials=A, P=4, n=1000, d=512, out=None, w=A, E=64, logits=None,
                                 K=8, H=4, renorm=1, idx=A, weights=None, rc=None, ec=None,
                                 local=None, s=None), **k)
    call = lambda a: f(*a.values())
    assert call(args(n=-1)) == SHAPE
    assert call(args(H=3)) == SHAPE             # E % H
    assert call(args(K=6)) == SHAPE             # K % H
    assert call(args(E=8, H=4, K=12)) == SHAPE  # K/H > E/H
    assert call(args(d=12)) == SHAPE
    assert call(args(P=3)) == UNSUP
    assert call(args(d=520)) == UNSUP           # d % 128
    assert call(args(E=168, H=4)) == UNSUP      # more than 160 columns
    assert call(args(K=20, H=4)) == UNSUP       # K > 16
    assert call(args(idx=None)) == NULL
    assert call(args(partials=None)) == NULL
    assert call(args(ec=A)) == NULL             # the count needs local
    assert call(args(ec=A, local=A)) == NULL    # and row_cluster
    assert call(args(out=MIS)) == ALIGN
    assert call(args(n=0)) == OK


def test_est_out_topk_errors(L):
    f = L.route_est_out_topk_packed
    args = lambda **k: dict(dict(h=A, n=100, hd=512, w2p=A, b2=None, E=128, K=8, logits=None, idx=A,
                                 truth=None, hits=None, s=None), **k)
    call = lambda a: f(*a.values())
    assert call(args(n=-1)) == SHAPE
    assert call(args(K=129)) == SHAPE
    assert call(args(hd=12)) == SHAPE
    assert call(args(hd=640)) == UNSUP
    assert call(args(E=257, K=8)) == UNSUP
    assert call(args(K=17)) == UNSUP
    assert call(args(idx=None)) == NULL
    assert call(args(truth=A)) == NULL          # truth and hits together
    assert call(args(h=MIS)) == ALIGN
    assert call(args(n=0)) == OK


def test_permute_and_combine_errors(L):
    ws = L.moe_permute_workspace_size(1000, 6, 160)
    assert ws > 0
    f = L.moe_permute
    assert f(A, 1000, 6, 160, 1, A, 64, A, A, A, None, A, ws, None, None) == NULL  # src w/o disp
    assert f(A, 1000, 6, 160, 1, A, 64, A, A, A, A, A, ws - 4, None, None) == WS
    assert f(A, 1000, 6, 160, 4, A, 64, A, A, A, A, A, ws, None, None) == SHAPE   # K % H
    assert f(A, 1000, 17, 160, 1, None, 0, A, A, A, None, A, ws, None, None) == UNSUP
    assert f(A, 1000, 6, 160, 1, A, 64, A, A, A, MIS, A, ws, None, None) == ALIGN
    g = L.moe_combine
    assert g(A, A, A, 100, 6, 64, None, A, 2, None, None) == SHAPE     # out_dtype
    assert g(A, A, A, 100, 6, 60, None, A, 0, None, None) == SHAPE
    assert g(A, A, None, 100, 6, 64, None, A, 0, None, None) == NULL
    assert g(A, A, A, 100, 17, 64, None, A, 0, None, None) == UNSUP
    assert g(A, A, A, 0, 6, 64, None, A, 0, None, None) == OK
    h = L.moe_combine_gather
    assert h(A, A, A, 100, 6, 64, None, A, 0, None, None) == NULL      # in_row
    assert h(A, A, A, 100, 6, 64, A, A, 2, None, None) == SHAPE
    assert h(A, A, A, 100, 17, 64, A, A, 0, None, None) == UNSUP
    assert h(A, A, A, 100, 6, 64, A, MIS, 0, None, None) == ALIGN
    assert h(A, A, A, 0, 6, 64, None, A, 0, None, None) == OK


def test_permute_noalloc_errors(L):
    """The host checks of moe_permute, all made before the static scratch is
    looked up (so none of these reaches the GPU)."""
    f = L.moe_permute_noalloc
    assert f(A, 1000, 6, 160, 1, A, 64, A, A, A, None, None, None) == NULL   # src w/o disp
    assert f(A, 1000, 6, 160, 1, A, 64, None, A, A, A, None, None) == NULL   # no offsets
    assert f(A, 1000, 6, 160, 4, A, 64, A, A, A, A, None, None) == SHAPE    # K % H
    assert f(A, 1000, 6, 160, 1, A, 60, A, A, A, A, None, None) == SHAPE    # d % 8
    assert f(A, 1000, 17, 160, 1, None, 0, A, A, A, None, None, None) == UNSUP
    assert f(A, 1000, 6, 2000, 1, None, 0, A, A, A, None, None, None) == UNSUP
    assert f(A, 1000, 6, 160, 1, A, 64, A, A, A, MIS, None, None) == ALIGN
    # the 512 KiB table covers the largest supported sort (n*K < 2^31, E <= 1024)
    assert L.moe_permute_workspace_size((1 << 31) // 16 - 1, 16, 1024) <= 512 * 1024
    assert L.moe_permute_workspace_size((1 << 31) // 16 - 1, 16, 1024) == 512 * 1024


def test_predict_lut_errors(L):
    f = L.route_predict
    assert f(A, 10, A, A, 100, None, A, A, 8, 128, A, None, None) == NULL   # conf w/o prev2
    assert f(A, 10, A, None, 100, None, None, None, 300, 128, A, None, None) == UNSUP
    assert f(A, -1, A, None, 100, None, None, None, 8, 128, A, None, None) == SHAPE
    assert f(A, 0, A, None, 100, None, None, None, 8, 128, A, None, None) == OK
    g = L.route_lut_build
    assert g(A, 10, A, A, 17, A, 8, 4, A, None, 100, None, None) == UNSUP
    assert g(A, 10, None, A, 2, A, 8, 4, A, None, 100, None, None) == NULL


def test_predictor_errors(L):
    f = L.route_qhidden
    assert f(A, A, None, None, 10, 16384, ctypes.c_float(1e-5), A, None) == UNSUP
    assert f(A, A, None, None, 10, 64, ctypes.c_float(-1.0), A, None) == SHAPE
    assert f(A, None, None, None, 10, 64, ctypes.c_float(1e-5), A, None) == NULL
    assert f(A, A, None, None, 10, 64, ctypes.c_float(1e-5), MIS, None) == ALIGN
    need = L.route_estimator_workspace_size(100, 512)
    assert need >= 100 * 512 * 2
    g = L.route_estimator
    assert g(A, 100, 64, A, A, 512, A, A, 128, A, A, need - 1, None) == WS
    assert g(A, 100, 64, A, A, 8192, A, A, 128, A, A, need, None) == UNSUP
    assert L.lar_count(A, 10, 17, 1, A, A, 8, A, None) == UNSUP
    assert L.lar_count(A, 10, 4, 3, A, A, 8, A, None) == SHAPE
    assert L.hit_count(A, None, 10, 8, A, None) == NULL
    assert L.hit_count(A, A, 10, 17, A, None) == UNSUP


def test_workspace_sizes_monotone(L):
    a = L.srs_shuffle_workspace_size(1000, 8)
    b = L.srs_shuffle_workspace_size(100000, 8)
    assert b > a > 0
    assert L.srs_shuffle_workspace_size(-1, 8) == 0
    assert L.moe_permute_workspace_size(16384, 6, 160) < L.moe_permute_workspace_size(32768, 8, 160)
    assert L.moe_permute_workspace_size(10, 2, 2000) == 0


def test_eg_errors(L):
    # eg_profile(tok, idx, n, K, row_of_id, vocab, U, E, counts, freq, err, s)
    f = L.eg_profile
    assert f(A, A, -1, 2, A, 10, 4, 8, A, A, None, None) == SHAPE
    assert f(A, A, 10, 2, A, 10, 4, 2000, A, A, None, None) == UNSUP
    assert f(None, A, 10, 2, A, 10, 4, 8, A, A, None, None) == NULL
    assert f(None, None, 0, 2, None, 10, 4, 8, None, None, None, None) == OK
    # eg_sample(P, E, G, B, seed, iter, place, s)
    f = L.eg_sample
    assert f(A, 10, 4, 8, 0, 0, A, None) == SHAPE      # E % 4
    assert f(A, 16, 3, 8, 0, 0, A, None) == SHAPE      # E % G
    assert f(A, 64, 64, 8, 0, 0, A, None) == UNSUP     # G > 32
    assert f(A, 16, 4, 2000, 0, 0, A, None) == UNSUP   # B > 1024
    assert f(None, 16, 4, 8, 0, 0, A, None) == NULL
    # eg_score(counts, freq, U, E, G, place, B, local, load, ws, ws_bytes, err, s)
    f = L.eg_score
    need = L.eg_score_workspace_size(100, 16, 4, 8)
    assert need > 0 and L.eg_score_workspace_size(100, 15, 4, 8) == 0
    assert f(A, A, 100, 16, 4, A, 8, A, A, A, need - 1, None, None) == WS
    assert f(A, A, 100, 16, 4, A, 8, A, A, MIS, need, None, None) == WS
    assert f(A, A, 100, 16, 4, None, 8, A, A, A, need, None, None) == NULL
    assert f(A, A, 100, 18, 4, A, 8, A, A, A, need, None, None) == SHAPE
    # eg_update(local, load, place, B, E, G, total, tokens, theta, n_elite, alpha, P, bJ, bp, J, s)
    f = L.eg_update
    assert f(A, A, A, 8, 16, 4, 100, 50, 0.0, 0, 0.5, A, A, A, None, None) == SHAPE
    assert f(A, A, A, 8, 16, 4, 100, 50, 0.0, 9, 0.5, A, A, A, None, None) == SHAPE
    assert f(A, A, A, 8, 16, 4, 0, 50, 0.0, 1, 0.5, A, A, A, None, None) == SHAPE
    assert f(A, A, None, 8, 16, 4, 100, 50, 0.0, 1, 0.5, A, A, A, None, None) == NULL
    # eg_init(P, E, G, best_J, s)
    assert L.eg_init(A, 16, 5, A, None) == SHAPE
    assert L.eg_init(None, 16, 4, A, None) == NULL


def test_estfit_errors(L):
    f = L.route_est_hidden
    assert f(A, 10, 60, A, A, 64, A, None) == SHAPE
    assert f(A, 10, 64, A, A, 8192, A, None) == UNSUP
    assert f(None, 10, 64, A, A, 64, A, None) == NULL
    assert f(MIS, 10, 64, A, A, 64, A, None) == ALIGN
    assert f(None, 0, 64, None, None, 64, None, None) == OK
    need = L.est_fit_gram_workspace_size(100, 64, 8)
    assert need > 0 and L.est_fit_gram_workspace_size(100, 0, 8) == 0
    f = L.est_fit_gram
    assert f(A, A, 0, 64, 8, A, A, A, need, None) == SHAPE
    assert f(A, A, 100, 64, 8, A, A, A, need - 1, None) == WS
    assert f(A, A, 100, 5000, 8, A, A, A, need, None) == UNSUP
    assert f(None, A, 100, 64, 8, A, A, A, need, None) == NULL
    f = L.est_fit_solve
    assert f(A, A, 0, 8, 0.1, None, None) == SHAPE
    assert f(A, A, 65, 8, -1.0, None, None) == SHAPE
    assert f(A, A, 5000, 8, 0.1, None, None) == UNSUP
    assert f(None, A, 65, 8, 0.1, None, None) == NULL
    assert L.est_fit_weights(A, 0, 8, A, A, None) == SHAPE
    assert L.est_fit_weights(None, 64, 8, A, A, None) == NULL


def test_prefetch_errors(L):
    p, c, v = L.prefetch_plan, L.prefetch_copy, L.prefetch_coverage
    assert p(A, -1, 8, 128, 8, A, A, None, None) == SHAPE
    assert p(A, 4, 0, 128, 8, A, A, None, None) == SHAPE
    assert p(A, 4, 8, 128, 0, A, A, None, None) == SHAPE
    assert p(A, 4, 8, 128, 129, A, A, None, None) == SHAPE     # C > E
    assert p(A, 4, 8, 1025, 8, A, A, None, None) == UNSUP
    assert p(None, 4, 8, 128, 8, A, A, None, None) == NULL
    assert p(A, 4, 8, 128, 8, None, A, None, None) == NULL
    assert c(A, 0, 4096, A, 8, A, None, None) == SHAPE
    assert c(A, 128, -16, A, 8, A, None, None) == SHAPE
    assert c(A, 2048, 4096, A, 8, A, None, None) == UNSUP
    assert c(A, 128, 4100, A, 8, A, None, None) == ALIGN
    assert c(MIS, 128, 4096, A, 8, A, None, None) == ALIGN
    assert c(A, 128, 4096, A, 8, MIS, None, None) == ALIGN
    assert c(None, 128, 4096, A, 8, A, None, None) == NULL
    assert c(A, 128, 0, A, 8, A, None, None) == OK           # nothing to copy
    assert v(A, -1, 8, 128, A, 8, A, A, A, None, None) == SHAPE
    assert v(A, 4, 8, 2048, A, 8, A, A, A, None, None) == UNSUP
    assert v(A, 4, 8, 128, A, 8, None, A, A, None, None) == NULL
    assert v(A, 4, 8, 128, A, 8, A, None, A, None, None) == NULL


def test_prefetch_issue_checks_the_host_list_first(L):
    f = L.prefetch_issue
    lst = (ctypes.c_int32 * 4)(0, 3, -1, 2)
    bad_hi = (ctypes.c_int32 * 4)(0, 3, 4, 2)     # 4 >= E
    bad_lo = (ctypes.c_int32 * 4)(0, -2, 1, 2)    # only -1 marks an empty slot
    addr = lambda a: ctypes.cast(a, ctypes.c_void_p).value
    assert f(A, 4, 4096, addr(bad_hi), 4, A, None) == SHAPE
    assert f(A, 4, 4096, addr(bad_lo), 4, A, None) == SHAPE
    assert f(A, 0, 4096, addr(lst), 4, A, None) == SHAPE
    assert f(A, 4, -1, addr(lst), 4, A, None) == SHAPE
    assert f(A, 4, 4096, addr(lst), 0, A, None) == SHAPE
    assert f(None, 4, 4096, addr(lst), 4, A, None) == NULL
    assert f(A, 4, 4096, None, 4, A, None) == NULL
    assert f(A, 4, 4096, addr(lst), 4, None, None) == NULL
    assert f(A, 4, 0, addr(lst), 4, A, None) == OK          # nothing to copy


def test_qgate_errors(L):
    f = L.route_qgate
    assert f(A, A, None, None, -1, 2048, 1e-5, A, 128, A, None) == SHAPE
    assert f(A, A, None, None, 10, 2044, 1e-5, A, 128, A, None) == SHAPE
    assert f(A, A, None, None, 10, 2048, -1.0, A, 128, A, None) == SHAPE
    assert f(A, A, None, None, 10, 2048, 1e-5, A, 0, A, None) == SHAPE
    assert f(A, A, None, None, 10, 512, 1e-5, A, 128, A, None) == UNSUP
    assert f(A, A, None, None, 10, 2048, 1e-5, A, 1025, A, None) == UNSUP
    assert f(None, A, None, None, 10, 2048, 1e-5, A, 128, A, None) == NULL
    assert f(A, A, None, None, 10, 2048, 1e-5, None, 128, A, None) == NULL
    assert f(MIS, A, None, None, 10, 2048, 1e-5, A, 128, A, None) == ALIGN
    assert f(A, A, MIS, None, 10, 2048, 1e-5, A, 128, A, None) == ALIGN
    assert f(A, A, None, None, 0, 2048, 1e-5, A, 128, A, None) == OK     # n = 0 is a no-op


def test_qgate_topk_errors(L):
    f = L.route_qgate_topk
    assert f(A, A, None, None, 10, 2048, 1e-5, A, 128, 0, None, A, None, None, None) == SHAPE
    assert f(A, A, None, None, 10, 2048, 1e-5, A, 4, 5, None, A, None, None, None) == SHAPE     # K > E
    assert f(A, A, None, None, 10, 2048, 1e-5, A, 257, 8, None, A, None, None, None) == UNSUP
    assert f(A, A, None, None, 10, 2048, 1e-5, A, 128, 17, None, A, None, None, None) == UNSUP
    assert f(A, A, None, None, 10, 512, 1e-5, A, 128, 8, None, A, None, None, None) == UNSUP
    assert f(A, A, None, None, 10, 2048, 1e-5, A, 128, 8, None, None, None, None, None) == NULL
    assert f(A, A, None, None, 10, 2048, 1e-5, A, 128, 8, None, A, A, None, None) == NULL  # truth without hits
    assert f(A, A, None, None, 10, 2048, 1e-5, A, 128, 8, None, A, None, A, None) == NULL  # hits without truth
    assert f(A, A, None, None, 0, 2048, 1e-5, A, 128, 8, None, A, None, None, None) == OK


def test_qgate_packed_errors(L):
    """The packed form's checks are the unpacked one's; packing takes d % 32 == 0."""
    f = L.route_qgate_topk_packed
    assert f(A, A, None, None, 10, 2048, 1e-5, A, 128, 0, None, A, None, None, None) == SHAPE
    assert f(A, A, None, None, 10, 2048, 1e-5, A, 257, 8, None, A, None, None, None) == UNSUP
    assert f(A, A, None, None, 10, 512, 1e-5, A, 128, 8, None, A, None, None, None) == UNSUP
    assert f(A, A, None, None, 10, 2048, 1e-5, None, 128, 8, None, A, None, None, None) == NULL
    assert f(A, A, None, None, 10, 2048, 1e-5, MIS, 128, 8, None, A, None, None, None) == ALIGN
    assert f(A, A, None, None, 0, 2048, 1e-5, A, 128, 8, None, A, None, None, None) == OK
    g = L.route_gate_pack
    assert g(A, 128, 2040, A, None) == SHAPE
    assert g(A, 0, 2048, A, None) == SHAPE
    assert g(A, 1025, 2048, A, None) == UNSUP
    assert g(None, 128, 2048, A, None) == NULL
    assert g(A, 128, 2048, MIS, None) == ALIGN
    assert L.route_gate_packed_size(128, 2048) == 128 * 2048 * 2
    assert L.route_gate_packed_size(100, 1024) == 112 * 1024 * 2   # rows padded to 16
    assert L.route_gate_packed_size(8, 100) == 0

