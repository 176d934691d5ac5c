"""MI355X-native MoE token routing and dispatch.

A thin ctypes binding over ``libroute.so`` (declared in ``include/route.h``).
Every function here only marshals arguments: it checks dtypes, devices and
contiguity of torch tensors, passes their device pointers and the current
HIP stream to the C entry point of the same name, and raises ``RouteError``
on a non-zero status. All arithmetic runs in the library's HIP kernels; there
is no fallback path. PyTorch is used only for device memory and streams.

Outputs may be passed in (``out=``-style keyword arguments) or are allocated
with ``torch.empty`` on the input's device. Workspaces likewise.
"""

from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "RouteError", "lib", "library_path",
    "route_predict", "route_predict_sort", "route_predict_sort_workspace_size", "route_lut_build",
    "srs_shuffle", "srs_route_sorted", "srs_predict_route", "srs_predict_route_dispatch",
    "srs_predict_route_dispatch_workspace_size", "srs_route_grouped",
    "srs_shuffle_gate", "srs_shuffle_route", "route_gate", "route_topk",
    "lar_count", "moe_permute", "moe_permute_noalloc", "moe_combine", "moe_combine_gather", "route_qhidden",
    "route_estimator",
    "hit_count", "srs_shuffle_workspace_size", "moe_permute_workspace_size",
    "route_estimator_workspace_size", "eg_profile", "eg_init", "eg_sample",
    "eg_score_workspace_size", "eg_score", "eg_update", "route_est_hidden",
    "est_fit_gram_workspace_size", "est_fit_gram", "est_fit_solve", "est_fit_weights",
    "prefetch_plan", "prefetch_copy", "prefetch_coverage", "prefetch_issue", "route_qgate",
    "route_qgate_topk", "route_gate_packed_size", "route_gate_pack", "route_qgate_topk_packed",
    "route_est_out_topk_packed", "route_qest_hidden_packed", "route_qest_topk_packed",
    "EXPORTS",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
# ROUTE_LIBRARY names another build of the same library (the host-sanitizer
# build the ABI tests can run against); unset, the in-tree libroute.so loads
_LIB_PATH = os.environ.get("ROUTE_LIBRARY") or os.path.join(_HERE, "libroute.so")

# status codes and device error bits (include/route.h)
ROUTE_OK = 0
EBIT_TOKEN_RANGE, EBIT_DEST_RANGE, EBIT_EXPERT_RANGE, EBIT_INDEX_RANGE = 1, 2, 4, 8
EBIT_VALUE_RANGE, EBIT_SYNC = 16, 32

_p, _i32, _i64, _sz, _f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float
_u64, _f64 = ctypes.c_uint64, ctypes.c_double

# name -> (restype, argtypes), in the header's order
EXPORTS = {
    "route_status_str": (ctypes.c_char_p, [ctypes.c_int]),
    "route_predict": (ctypes.c_int, [_p, _i64, _p, _p, _i32, _p, _p, _p, _i32, _i32, _p, _p, _p]),
    "route_predict_sort": (ctypes.c_int, [_p, _i64, _p, _p, _i32, _p, _p, _p, _i32, _i32, _p, _p,
                                          _p, _p, _p, _p, _sz, _p, _p]),
    "route_predict_sort_workspace_size": (_sz, [_i64, _i32]),
    "route_lut_build": (ctypes.c_int, [_p, _i64, _p, _p, _i32, _p, _i32, _i32, _p, _p, _i32, _p, _p]),
    "srs_shuffle": (ctypes.c_int, [_p, _i32, _i64, _i32, _p, _i32, _p, _p, _p, _p, _p, _p, _sz, _p, _p]),
    "srs_shuffle_gate": (ctypes.c_int, [_p, _i32, _i64, _i32, _p, _i32, _p, _p, _p, _p, _p,
                                        _p, _i32, _p, _p, _sz, _p, _p]),
    "srs_shuffle_route": (ctypes.c_int, [_p, _i32, _i64, _i32, _p, _i32, _p, _p, _p, _p, _p,
                                         _p, _i32, _p, _i32, _i32, _p, _p, _p, _p, _p, _sz, _p,
                                         _p]),
    "srs_route_sorted": (ctypes.c_int, [_p, _i32, _i64, _i32, _p, _p, _p, _p, _i32, _p, _i32, _i32,
                                        _p, _p, _p, _p, _p]),
    "srs_predict_route": (ctypes.c_int, [_p, _i64, _p, _p, _i32, _p, _p, _p, _i32, _i32, _p, _i32,
                                         _i32, _p, _i32, _i32, _i32, _p, _p, _p, _p, _p, _p, _p,
                                         _p, _p, _p, _p, _p, _p]),
    "srs_predict_route_dispatch": (ctypes.c_int, [_p, _i64, _p, _p, _i32, _p, _p, _p, _i32, _i32,
                                                  _p, _i32, _i32, _p, _i32, _i32, _i32, _p, _p,
                                                  _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p,
                                                  _p, _p, _sz, _p, _p]),
    "srs_predict_route_dispatch_workspace_size": (_sz, [_i64, _i32, _i32]),
    "srs_route_grouped": (ctypes.c_int, [_p, _i32, _i64, _i32, _p, _p, _i32, _p, _i32, _i32, _i32,
                                         _p, _p, _p, _p, _p, _p]),
    "srs_shuffle_workspace_size": (_sz, [_i64, _i32]),
    "route_gate": (ctypes.c_int, [_p, _i64, _i32, _p, _i32, _p, _p]),
    "route_topk": (ctypes.c_int, [_p, _i64, _i32, _i32, _i32, _i32, _p, _p, _p]),
    "lar_count": (ctypes.c_int, [_p, _i64, _i32, _i32, _p, _p, _i32, _p, _p]),
    "moe_permute": (ctypes.c_int, [_p, _i64, _i32, _i32, _i32, _p, _i32, _p, _p, _p, _p, _p, _sz, _p, _p]),
    "moe_permute_workspace_size": (_sz, [_i64, _i32, _i32]),
    "moe_permute_noalloc": (ctypes.c_int, [_p, _i64, _i32, _i32, _i32, _p, _i32, _p, _p, _p, _p, _p,
                                           _p]),
    "moe_combine": (ctypes.c_int, [_p, _p, _p, _i64, _i32, _i32, _p, _p, _i32, _p, _p]),
    "moe_combine_gather": (ctypes.c_int, [_p, _p, _p, _i64, _i32, _i32, _p, _p, _i32, _p, _p]),
    "route_qhidden": (ctypes.c_int, [_p, _p, _p, _p, _i64, _i32, _f32, _p, _p]),
    "route_qgate": (ctypes.c_int, [_p, _p, _p, _p, _i64, _i32, _f32, _p, _i32, _p, _p]),
    "route_qgate_topk": (ctypes.c_int, [_p, _p, _p, _p, _i64, _i32, _f32, _p, _i32, _i32, _p, _p,
                                        _p, _p, _p]),
    "route_gate_packed_size": (_sz, [_i32, _i32]),
    "route_gate_pack": (ctypes.c_int, [_p, _i32, _i32, _p, _p]),
    "route_qgate_topk_packed": (ctypes.c_int, [_p, _p, _p, _p, _i64, _i32, _f32, _p, _i32, _i32, _p,
                                               _p, _p, _p, _p]),
    "route_est_out_topk_packed": (ctypes.c_int, [_p, _i64, _i32, _p, _p, _i32, _i32, _p, _p, _p,
                                                 _p, _p]),
    "route_qest_hidden_packed": (ctypes.c_int, [_p, _p, _p, _p, _i64, _i32, _f32, _p, _p, _i32,
                                                _p, _p]),
    "route_qest_topk_packed": (ctypes.c_int, [_p, _p, _p, _p, _i64, _i32, _f32, _p, _p, _i32, _p,
                                              _p, _i32, _i32, _p, _p, _p, _p, _p]),
    "route_estimator": (ctypes.c_int, [_p, _i64, _i32, _p, _p, _i32, _p, _p, _i32, _p, _p, _sz, _p]),
    "route_estimator_workspace_size": (_sz, [_i64, _i32]),
    "hit_count": (ctypes.c_int, [_p, _p, _i64, _i32, _p, _p]),
    "eg_profile": (ctypes.c_int, [_p, _p, _i64, _i32, _p, _i32, _i32, _i32, _p, _p, _p, _p]),
    "eg_init": (ctypes.c_int, [_p, _i32, _i32, _p, _p]),
    "eg_sample": (ctypes.c_int, [_p, _i32, _i32, _i32, _u64, _i32, _p, _p]),
    "eg_score_workspace_size": (_sz, [_i32, _i32, _i32, _i32]),
    "eg_score": (ctypes.c_int, [_p, _p, _i32, _i32, _i32, _p, _i32, _p, _p, _p, _sz, _p, _p]),
    "eg_update": (ctypes.c_int, [_p, _p, _p, _i32, _i32, _i32, _i64, _i64, _f64, _i32, _f64,
                                 _p, _p, _p, _p, _p]),
    "route_est_hidden": (ctypes.c_int, [_p, _i64, _i32, _p, _p, _i32, _p, _p]),
    "est_fit_gram_workspace_size": (_sz, [_i64, _i32, _i32]),
    "est_fit_gram": (ctypes.c_int, [_p, _p, _i64, _i32, _i32, _p, _p, _p, _sz, _p]),
    "est_fit_solve": (ctypes.c_int, [_p, _p, _i32, _i32, _f64, _p, _p]),
    "est_fit_weights": (ctypes.c_int, [_p, _i32, _i32, _p, _p, _p]),
    "prefetch_plan": (ctypes.c_int, [_p, _i64, _i32, _i32, _i32, _p, _p, _p, _p]),
    "prefetch_copy": (ctypes.c_int, [_p, _i32, _i64, _p, _i32, _p, _p, _p]),
    "prefetch_issue": (ctypes.c_int, [_p, _i32, _i64, _p, _i32, _p, _p]),
    "prefetch_coverage": (ctypes.c_int, [_p, _i64, _i32, _i32, _p, _i32, _p, _p, _p, _p, _p]),
}


class RouteError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn}: status {status} ({_status_str(status)})")


_lib = None


def library_path() -> str:
    return _LIB_PATH


def lib() -> ctypes.CDLL:
    """The loaded libroute.so. Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(
                f"{_LIB_PATH} is missing: build it with "
                "`python -m token_routing_speculation_amd.build` (no fallback exists)")
        handle = ctypes.CDLL(_LIB_PATH)
        for name, (res, args) in EXPORTS.items():
            f = getattr(handle, name)
            f.restype = res
            f.argtypes = args
        _lib = handle
    return _lib


def _status_str(status: int) -> str:
    try:
        return lib().route_status_str(status).decode()
    except Exception:  # pragma: no cover - only while the library is unusable
        return "?"


def _call(name: str, *args) -> None:
    st = getattr(lib(), name)(*args)
    if st != ROUTE_OK:
        raise RouteError(name, st)


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _dev(t: torch.Tensor, dtype, name: str, numel: int | None = None) -> int:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU device")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} must hold {numel} elements, has {t.numel()}")
    return t.data_ptr()


def _opt(t, dtype, name, numel=None):
    return None if t is None else _dev(t, dtype, name, numel)


def _empty(shape, dtype, like: torch.Tensor):
    return torch.empty(shape, dtype=dtype, device=like.device)


def _bf16(t: torch.Tensor) -> torch.dtype:
    # bf16 rows may be given as torch.bfloat16 or as their int16 bit patterns
    return t.dtype if t.dtype in (torch.bfloat16, torch.int16) else torch.bfloat16


# ------------------------------------------------------------------ entry points

def route_predict(tok, lut, G, conf=None, prev2=None, prev1=None, ngram=None, conf_thr=128,
                  dest=None, err=None, stream=None):
    n = tok.numel()
    dest = _empty((n,), torch.uint8, tok) if dest is None else dest
    fb = conf is not None
    _call("route_predict", _dev(tok, torch.int32, "tok"), n, _dev(lut, torch.uint8, "lut"),
          _opt(conf, torch.uint8, "conf"), lut.numel(),
          _opt(prev2, torch.uint8, "prev2", n if fb else None),
          _opt(prev1, torch.uint8, "prev1", n if fb else None),
          _opt(ngram, torch.uint8, "ngram", G * G if fb else None), G, conf_thr,
          _dev(dest, torch.uint8, "dest", n), _opt(err, torch.int32, "err", 1), _stream(stream))
    return dest


def route_predict_sort_workspace_size(n: int, G: int) -> int:
    return int(lib().route_predict_sort_workspace_size(n, G))


def route_predict_sort(tok, lut, G, conf=None, prev2=None, prev1=None, ngram=None, conf_thr=128,
                       dest=None, offsets=None, row_of_src=None, src_of_row=None,
                       row_cluster=None, ws=None, err=None, stream=None):
    """route_predict and the stable sort of its clusters in one go: returns
    (dest, offsets, row_of_src, src_of_row, row_cluster)."""
    n = tok.numel()
    e = lambda shape, dt: _empty(shape, dt, tok)
    dest = e((n,), torch.uint8) if dest is None else dest
    offsets = e((G + 1,), torch.int32) if offsets is None else offsets
    row_of_src = e((n,), torch.int32) if row_of_src is None else row_of_src
    src_of_row = e((n,), torch.int32) if src_of_row is None else src_of_row
    row_cluster = e((n,), torch.uint8) if row_cluster is None else row_cluster
    need = route_predict_sort_workspace_size(n, G)
    ws = e((max(need, 1),), torch.uint8) if ws is None else ws
    fb = conf is not None
    _call("route_predict_sort", _dev(tok, torch.int32, "tok"), n, _dev(lut, torch.uint8, "lut"),
          _opt(conf, torch.uint8, "conf"), lut.numel(),
          _opt(prev2, torch.uint8, "prev2", n if fb else None),
          _opt(prev1, torch.uint8, "prev1", n if fb else None),
          _opt(ngram, torch.uint8, "ngram", G * G if fb else None), G, conf_thr,
          _dev(dest, torch.uint8, "dest", n), _dev(offsets, torch.int32, "offsets", G + 1),
          _dev(row_of_src, torch.int32, "row_of_src", n),
          _dev(src_of_row, torch.int32, "src_of_row", n),
          _opt(row_cluster, torch.uint8, "row_cluster", n), _dev(ws, torch.uint8, "ws"),
          ws.numel(), _opt(err, torch.int32, "err", 1), _stream(stream))
    return dest, offsets, row_of_src, src_of_row, row_cluster


def route_lut_build(ids, idx, w, expert_cluster, G, lut, conf=None, err=None, stream=None):
    n, K = idx.shape
    _call("route_lut_build", _dev(ids, torch.int32, "ids", n), n, _dev(idx, torch.int32, "idx"),
          _dev(w, torch.float32, "w", n * K), K, _dev(expert_cluster, torch.uint8, "expert_cluster"),
          expert_cluster.numel(), G, _dev(lut, torch.uint8, "lut"),
          _opt(conf, torch.uint8, "conf", lut.numel()), lut.numel(),
          _opt(err, torch.int32, "err", 1), _stream(stream))
    return lut, conf


def srs_shuffle_workspace_size(n: int, G: int) -> int:
    return int(lib().srs_shuffle_workspace_size(n, G))


def srs_shuffle(partials, dest, G, out=None, offsets=None, row_of_src=None, src_of_row=None,
                row_cluster=None, maps=True, ws=None, err=None, stream=None):
    """partials [P][n][d] bf16 -> (out [n][d], offsets [G+1], row_of_src, src_of_row, row_cluster)."""
    P, n, d = partials.shape
    bt = _bf16(partials)
    out = _empty((n, d), bt, partials) if out is None else out
    offsets = _empty((G + 1,), torch.int32, partials) if offsets is None else offsets
    if maps:
        row_of_src = _empty((n,), torch.int32, partials) if row_of_src is None else row_of_src
        src_of_row = _empty((n,), torch.int32, partials) if src_of_row is None else src_of_row
        row_cluster = _empty((n,), torch.uint8, partials) if row_cluster is None else row_cluster
    need = srs_shuffle_workspace_size(n, G)
    ws = _empty((max(need, 1),), torch.uint8, partials) if ws is None else ws
    _call("srs_shuffle", _dev(partials, bt, "partials"), P, n, d,
          _opt(dest, torch.uint8, "dest", n), G, _dev(out, bt, "out", n * d),
          _dev(offsets, torch.int32, "offsets", G + 1), _opt(row_of_src, torch.int32, "row_of_src", n),
          _opt(src_of_row, torch.int32, "src_of_row", n), _opt(row_cluster, torch.uint8, "row_cluster", n),
          _dev(ws, torch.uint8, "ws"), ws.numel(), _opt(err, torch.int32, "err", 1), _stream(stream))
    return out, offsets, row_of_src, src_of_row, row_cluster



def srs_shuffle_gate(partials, dest, G, w, out=None, logits=None, offsets=None, row_of_src=None,
                     src_of_row=None, row_cluster=None, maps=True, ws=None, err=None, stream=None):
    """srs_shuffle and route_gate on its output in one pass: returns
    (out, offsets, row_of_src, src_of_row, row_cluster, logits)."""
    P, n, d = partials.shape
    E = w.shape[0]
    bt = _bf16(partials)
    out = _empty((n, d), bt, partials) if out is None else out
    logits = _empty((n, E), torch.float32, partials) if logits is None else logits
    offsets = _empty((G + 1,), torch.int32, partials) if offsets is None else offsets
    if maps:
        row_of_src = _empty((n,), torch.int32, partials) if row_of_src is None else row_of_src
        src_of_row = _empty((n,), torch.int32, partials) if src_of_row is None else src_of_row
        row_cluster = _empty((n,), torch.uint8, partials) if row_cluster is None else row_cluster
    need = srs_shuffle_workspace_size(n, G)
    ws = _empty((max(need, 1),), torch.uint8, partials) if ws is None else ws
    _call("srs_shuffle_gate", _dev(partials, bt, "partials"), P, n, d,
          _opt(dest, torch.uint8, "dest", n), G, _dev(out, bt, "out", n * d),
          _dev(offsets, torch.int32, "offsets", G + 1), _opt(row_of_src, torch.int32, "row_of_src", n),
          _opt(src_of_row, torch.int32, "src_of_row", n), _opt(row_cluster, torch.uint8, "row_cluster", n),
          _dev(w, _bf16(w), "w", E * d), E, _dev(logits, torch.float32, "logits", n * E),
          _dev(ws, torch.uint8, "ws"), ws.numel(), _opt(err, torch.int32, "err", 1), _stream(stream))
    return out, offsets, row_of_src, src_of_row, row_cluster, logits

def srs_shuffle_route(partials, dest, G, w, K, renorm=1, expert_cluster=None, local=None,
                      out=None, logits=None, idx=None, weights=None, offsets=None, row_of_src=None,
                      src_of_row=None, row_cluster=None, maps=True, with_logits=True, ws=None,
                      err=None, stream=None):
    """srs_shuffle, then the router, top-K and the local activation count of
    every reduced row in one pass: returns (out, offsets, row_of_src,
    src_of_row, row_cluster, logits, idx, weights). ``local`` (uint64 as
    int64, accumulated) goes with ``expert_cluster``; ``with_logits=False``
    leaves the logits unwritten (None returned)."""
    P, n, d = partials.shape
    E = w.shape[0]
    bt = _bf16(partials)
    out = _empty((n, d), bt, partials) if out is None else out
    if with_logits and logits is None:
        logits = _empty((n, E), torch.float32, partials)
    idx = _empty((n, K), torch.int32, partials) if idx is None else idx
    weights = _empty((n, K), torch.float32, partials) if weights is None else weights
    offsets = _empty((G + 1,), torch.int32, partials) if offsets is None else offsets
    if maps:
        row_of_src = _empty((n,), torch.int32, partials) if row_of_src is None else row_of_src
        src_of_row = _empty((n,), torch.int32, partials) if src_of_row is None else src_of_row
        row_cluster = _empty((n,), torch.uint8, partials) if row_cluster is None else row_cluster
    need = srs_shuffle_workspace_size(n, G)
    ws = _empty((max(need, 1),), torch.uint8, partials) if ws is None else ws
    _call("srs_shuffle_route", _dev(partials, bt, "partials"), P, n, d,
          _opt(dest, torch.uint8, "dest", n), G, _dev(out, bt, "out", n * d),
          _dev(offsets, torch.int32, "offsets", G + 1), _opt(row_of_src, torch.int32, "row_of_src", n),
          _opt(src_of_row, torch.int32, "src_of_row", n), _opt(row_cluster, torch.uint8, "row_cluster", n),
          _dev(w, _bf16(w), "w", E * d), E, _opt(logits, torch.float32, "logits", n * E), K, renorm,
          _dev(idx, torch.int32, "idx", n * K), _opt(weights, torch.float32, "weights", n * K),
          _opt(expert_cluster, torch.uint8, "expert_cluster", E), _opt(local, torch.int64, "local", 1),
          _dev(ws, torch.uint8, "ws"), ws.numel(), _opt(err, torch.int32, "err", 1), _stream(stream))
    return out, offsets, row_of_src, src_of_row, row_cluster, logits, idx, weights


def srs_route_sorted(partials, row_of_src, w, K, renorm=1, dest=None, expert_cluster=None,
                     local=None, out=None, logits=None, idx=None, weights=None,
                     with_logits=True, stream=None):
    """srs_shuffle_route's row work for an order already made (row_of_src):
    returns (out, logits, idx, weights)."""
    P, n, d = partials.shape
    E = w.shape[0]
    bt = _bf16(partials)
    out = _empty((n, d), bt, partials) if out is None else out
    if with_logits and logits is None:
        logits = _empty((n, E), torch.float32, partials)
    idx = _empty((n, K), torch.int32, partials) if idx is None else idx
    weights = _empty((n, K), torch.float32, partials) if weights is None else weights
    _call("srs_route_sorted", _dev(partials, bt, "partials"), P, n, d,
          _dev(row_of_src, torch.int32, "row_of_src", n), _opt(dest, torch.uint8, "dest", n),
          _dev(out, bt, "out", n * d), _dev(w, _bf16(w), "w", E * d), E,
          _opt(logits, torch.float32, "logits", n * E), K, renorm,
          _dev(idx, torch.int32, "idx", n * K), _opt(weights, torch.float32, "weights", n * K),
          _opt(expert_cluster, torch.uint8, "expert_cluster", E), _opt(local, torch.int64, "local", 1),
          _stream(stream))
    return out, logits, idx, weights


def srs_predict_route(tok, lut, G, partials, w, K, renorm=1, conf=None, prev2=None, prev1=None,
                      ngram=None, conf_thr=128, expert_cluster=None, local=None, dest=None,
                      offsets=None, row_of_src=None, src_of_row=None, row_cluster=None, out=None,
                      logits=None, idx=None, weights=None, with_logits=True, err=None,
                      stream=None):
    """route_predict_sort + srs_route_sorted in one launch (small batches):
    returns (dest, offsets, row_of_src, src_of_row, row_cluster, out, logits,
    idx, weights)."""
    P, n, d = partials.shape
    E = w.shape[0]
    bt = _bf16(partials)
    e = lambda shape, dt: _empty(shape, dt, partials)
    dest = e((n,), torch.uint8) if dest is None else dest
    offsets = e((G + 1,), torch.int32) if offsets is None else offsets
    row_of_src = e((n,), torch.int32) if row_of_src is None else row_of_src
    src_of_row = e((n,), torch.int32) if src_of_row is None else src_of_row
    row_cluster = e((n,), torch.uint8) if row_cluster is None else row_cluster
    out = e((n, d), bt) if out is None else out
    if with_logits and logits is None:
        logits = e((n, E), torch.float32)
    idx = e((n, K), torch.int32) if idx is None else idx
    weights = e((n, K), torch.float32) if weights is None else weights
    fb = conf is not None
    _call("srs_predict_route", _dev(tok, torch.int32, "tok", n), n, _dev(lut, torch.uint8, "lut"),
          _opt(conf, torch.uint8, "conf"), lut.numel(),
          _opt(prev2, torch.uint8, "prev2", n if fb else None),
          _opt(prev1, torch.uint8, "prev1", n if fb else None),
          _opt(ngram, torch.uint8, "ngram", G * G if fb else None), G, conf_thr,
          _dev(partials, bt, "partials"), P, d, _dev(w, _bf16(w), "w", E * d), E, K, renorm,
          _dev(dest, torch.uint8, "dest", n), _dev(offsets, torch.int32, "offsets", G + 1),
          _dev(row_of_src, torch.int32, "row_of_src", n),
          _dev(src_of_row, torch.int32, "src_of_row", n),
          _opt(row_cluster, torch.uint8, "row_cluster", n), _dev(out, bt, "out", n * d),
          _opt(logits, torch.float32, "logits", n * E), _dev(idx, torch.int32, "idx", n * K),
          _opt(weights, torch.float32, "weights", n * K),
          _opt(expert_cluster, torch.uint8, "expert_cluster", E),
          _opt(local, torch.int64, "local", 1), _opt(err, torch.int32, "err", 1), _stream(stream))
    return dest, offsets, row_of_src, src_of_row, row_cluster, out, logits, idx, weights


def srs_predict_route_dispatch_workspace_size(n, G, E):
    return lib().srs_predict_route_dispatch_workspace_size(n, G, E)


def srs_predict_route_dispatch(tok, lut, G, partials, w, K, renorm=1, conf=None, prev2=None,
                               prev1=None, ngram=None, conf_thr=128, expert_cluster=None,
                               local=None, dest=None, offsets=None, row_of_src=None,
                               src_of_row=None, row_cluster=None, out=None, write_x=False,
                               logits=None, idx=None, weights=None, with_logits=True,
                               expert_offsets=None, slot_of_pair=None, pair_of_slot=None,
                               disp=None, ws=None, err=None, stream=None):
    """srs_predict_route + moe_permute (one group) in one launch: returns
    (dest, offsets, row_of_src, src_of_row, row_cluster, out, logits, idx,
    weights, expert_offsets, slot_of_pair, pair_of_slot, disp); out (the
    shuffled rows) only when given or write_x. ws must start zeroed (a
    fresh workspace is allocated zeroed) and is reused as it is left."""
    P, n, d = partials.shape
    E = w.shape[0]
    bt = _bf16(partials)
    e = lambda shape, dt: _empty(shape, dt, partials)
    dest = e((n,), torch.uint8) if dest is None else dest
    offsets = e((G + 1,), torch.int32) if offsets is None else offsets
    row_of_src = e((n,), torch.int32) if row_of_src is None else row_of_src
    src_of_row = e((n,), torch.int32) if src_of_row is None else src_of_row
    row_cluster = e((n,), torch.uint8) if row_cluster is None else row_cluster
    if out is None and write_x:
        out = e((n, d), bt)
    if with_logits and logits is None:
        logits = e((n, E), torch.float32)
    idx = e((n, K), torch.int32) if idx is None else idx
    weights = e((n, K), torch.float32) if weights is None else weights
    expert_offsets = e((E + 1,), torch.int32) if expert_offsets is None else expert_offsets
    slot_of_pair = e((n * K,), torch.int32) if slot_of_pair is None else slot_of_pair
    pair_of_slot = e((n * K,), torch.int32) if pair_of_slot is None else pair_of_slot
    disp = e((n * K, d), bt) if disp is None else disp
    if ws is None:
        ws = torch.zeros((max(srs_predict_route_dispatch_workspace_size(n, G, E), 256),),
                         dtype=torch.uint8, device=partials.device)
    fb = conf is not None
    _call("srs_predict_route_dispatch", _dev(tok, torch.int32, "tok", n), n,
          _dev(lut, torch.uint8, "lut"), _opt(conf, torch.uint8, "conf"), lut.numel(),
          _opt(prev2, torch.uint8, "prev2", n if fb else None),
          _opt(prev1, torch.uint8, "prev1", n if fb else None),
          _opt(ngram, torch.uint8, "ngram", G * G if fb else None), G, conf_thr,
          _dev(partials, bt, "partials"), P, d, _dev(w, _bf16(w), "w", E * d), E, K, renorm,
          _dev(dest, torch.uint8, "dest", n), _dev(offsets, torch.int32, "offsets", G + 1),
          _dev(row_of_src, torch.int32, "row_of_src", n),
          _dev(src_of_row, torch.int32, "src_of_row", n),
          _opt(row_cluster, torch.uint8, "row_cluster", n), _opt(out, bt, "out", n * d),
          _opt(logits, torch.float32, "logits", n * E), _dev(idx, torch.int32, "idx", n * K),
          _dev(weights, torch.float32, "weights", n * K),
          _opt(expert_cluster, torch.uint8, "expert_cluster", E),
          _opt(local, torch.int64, "local", 1),
          _dev(expert_offsets, torch.int32, "expert_offsets", E + 1),
          _dev(slot_of_pair, torch.int32, "slot_of_pair", n * K),
          _dev(pair_of_slot, torch.int32, "pair_of_slot", n * K), _dev(disp, bt, "disp", n * K * d),
          _dev(ws, torch.uint8, "ws"), ws.numel(), _opt(err, torch.int32, "err", 1),
          _stream(stream))
    return (dest, offsets, row_of_src, src_of_row, row_cluster, out, logits, idx, weights,
            expert_offsets, slot_of_pair, pair_of_slot, disp)


def srs_route_grouped(partials, w, K, H, renorm=1, row_cluster=None, expert_cluster=None,
                      local=None, out=None, logits=None, idx=None, weights=None,
                      with_logits=True, stream=None):
    """The cross-group reduce, router, grouped top-K and per-group count in
    one kernel: returns (out, logits, idx, weights); out (the reduced rows)
    is written only when given."""
    P, n, d = partials.shape
    E = w.shape[0]
    bt = _bf16(partials)
    if with_logits and logits is None:
        logits = _empty((n, E), torch.float32, partials)
    idx = _empty((n, K), torch.int32, partials) if idx is None else idx
    weights = _empty((n, K), torch.float32, partials) if weights is None else weights
    _call("srs_route_grouped", _dev(partials, bt, "partials"), P, n, d,
          _opt(out, bt, "out", n * d), _dev(w, _bf16(w), "w", E * d), E,
          _opt(logits, torch.float32, "logits", n * E), K, H, renorm,
          _dev(idx, torch.int32, "idx", n * K), _opt(weights, torch.float32, "weights", n * K),
          _opt(row_cluster, torch.uint8, "row_cluster", n * H),
          _opt(expert_cluster, torch.uint8, "expert_cluster", E),
          _opt(local, torch.int64, "local", 1), _stream(stream))
    return out, logits, idx, weights


def route_gate(x, w, logits=None, stream=None):
    n, d = x.shape
    E = w.shape[0]
    logits = _empty((n, E), torch.float32, x) if logits is None else logits
    _call("route_gate", _dev(x, _bf16(x), "x"), n, d, _dev(w, _bf16(w), "w", E * d), E,
          _dev(logits, torch.float32, "logits", n * E), _stream(stream))
    return logits


def route_topk(logits, K, H=1, renorm=1, idx=None, weights=None, want_weights=True, stream=None):
    n, E = logits.shape
    idx = _empty((n, K), torch.int32, logits) if idx is None else idx
    if want_weights and weights is None:
        weights = _empty((n, K), torch.float32, logits)
    _call("route_topk", _dev(logits, torch.float32, "logits"), n, E, K, H, renorm,
          _dev(idx, torch.int32, "idx", n * K), _opt(weights, torch.float32, "weights", n * K),
          _stream(stream))
    return idx, weights


def lar_count(idx, H, row_cluster, expert_cluster, local, stream=None):
    n, K = idx.shape
    _call("lar_count", _dev(idx, torch.int32, "idx"), n, K, H,
          _dev(row_cluster, torch.uint8, "row_cluster", n * H),
          _dev(expert_cluster, torch.uint8, "expert_cluster"), expert_cluster.numel(),
          _dev(local, torch.int64, "local", 1), _stream(stream))
    return local


def moe_permute_workspace_size(n: int, K: int, E: int) -> int:
    return int(lib().moe_permute_workspace_size(n, K, E))


def moe_permute(idx, E, src=None, H=1, expert_offsets=None, slot_of_pair=None, pair_of_slot=None,
                disp=None, ws=None, err=None, stream=None):
    """idx [n][K]; src [H][n][d] bf16 (optional) -> offsets, slot_of_pair, pair_of_slot, disp."""
    n, K = idx.shape
    expert_offsets = _empty((E + 1,), torch.int32, idx) if expert_offsets is None else expert_offsets
    slot_of_pair = _empty((n * K,), torch.int32, idx) if slot_of_pair is None else slot_of_pair
    pair_of_slot = _empty((n * K,), torch.int32, idx) if pair_of_slot is None else pair_of_slot
    d = 0
    if src is not None:
        if src.dim() == 2:
            src = src.unsqueeze(0)
        if src.shape[0] != H or src.shape[1] != n:
            raise ValueError("src must be [H][n][d]")
        d = src.shape[2]
        disp = _empty((n * K, d), _bf16(src), idx) if disp is None else disp
    need = moe_permute_workspace_size(n, K, E)
    ws = _empty((max(need, 1),), torch.uint8, idx) if ws is None else ws
    bt = _bf16(src) if src is not None else torch.bfloat16
    _call("moe_permute", _dev(idx, torch.int32, "idx"), n, K, E, H, _opt(src, bt, "src"), d,
          _dev(expert_offsets, torch.int32, "expert_offsets", E + 1),
          _dev(slot_of_pair, torch.int32, "slot_of_pair", n * K),
          _dev(pair_of_slot, torch.int32, "pair_of_slot", n * K),
          _opt(disp, bt, "disp", n * K * d if src is not None else None),
          _dev(ws, torch.uint8, "ws"), ws.numel(), _opt(err, torch.int32, "err", 1), _stream(stream))
    return expert_offsets, slot_of_pair, pair_of_slot, disp


def moe_permute_noalloc(idx, E, src=None, H=1, expert_offsets=None, slot_of_pair=None,
                        pair_of_slot=None, disp=None, err=None, stream=None):
    """moe_permute on the library's static per-GPU scratch (no workspace). With
    every output passed in, nothing is allocated on either side of the call."""
    n, K = idx.shape
    expert_offsets = _empty((E + 1,), torch.int32, idx) if expert_offsets is None else expert_offsets
    slot_of_pair = _empty((n * K,), torch.int32, idx) if slot_of_pair is None else slot_of_pair
    pair_of_slot = _empty((n * K,), torch.int32, idx) if pair_of_slot is None else pair_of_slot
    d = 0
    if src is not None:
        if src.dim() == 2:
            src = src.unsqueeze(0)
        if src.shape[0] != H or src.shape[1] != n:
            raise ValueError("src must be [H][n][d]")
        d = src.shape[2]
        disp = _empty((n * K, d), _bf16(src), idx) if disp is None else disp
    bt = _bf16(src) if src is not None else torch.bfloat16
    _call("moe_permute_noalloc", _dev(idx, torch.int32, "idx"), n, K, E, H, _opt(src, bt, "src"), d,
          _dev(expert_offsets, torch.int32, "expert_offsets", E + 1),
          _dev(slot_of_pair, torch.int32, "slot_of_pair", n * K),
          _dev(pair_of_slot, torch.int32, "pair_of_slot", n * K),
          _opt(disp, bt, "disp", n * K * d if src is not None else None),
          _opt(err, torch.int32, "err", 1), _stream(stream))
    return expert_offsets, slot_of_pair, pair_of_slot, disp


def moe_combine(y, weights, slot_of_pair, out_row=None, out=None, out_dtype=torch.bfloat16,
                err=None, stream=None, in_row=None):
    """Weighted combine with the unshuffle: out[out_row[j]] = o[j] (moe_combine),
    or, given ``in_row`` instead, out[t] = o[in_row[t]] (moe_combine_gather)."""
    n, K = weights.shape
    d = y.shape[1]
    code = {torch.bfloat16: 0, torch.int16: 0, torch.float32: 1}[out.dtype if out is not None else out_dtype]
    if out is None:
        out = _empty((n, d), out_dtype, y)
    if in_row is not None and out_row is not None:
        raise ValueError("give out_row or in_row, not both")
    common = (_dev(y, _bf16(y), "y", n * K * d), _dev(weights, torch.float32, "weights"),
              _dev(slot_of_pair, torch.int32, "slot_of_pair", n * K), n, K, d)
    tail = (_dev(out, out.dtype, "out", n * d), code, _opt(err, torch.int32, "err", 1),
            _stream(stream))
    if in_row is not None:
        _call("moe_combine_gather", *common, _dev(in_row, torch.int32, "in_row", n), *tail)
    else:
        _call("moe_combine", *common, _opt(out_row, torch.int32, "out_row", n), *tail)
    return out


def route_qhidden(r, dvec, gamma=None, beta=None, eps=1e-5, q=None, stream=None):
    n, d = r.shape
    q = _empty((n, d), _bf16(r), r) if q is None else q
    _call("route_qhidden", _dev(r, _bf16(r), "r"), _dev(dvec, torch.float32, "dvec", d),
          _opt(gamma, torch.float32, "gamma", d), _opt(beta, torch.float32, "beta", d), n, d,
          float(eps), _dev(q, _bf16(r), "q", n * d), _stream(stream))
    return q


def route_qgate(r, dvec, w, gamma=None, beta=None, eps=1e-5, logits=None, stream=None):
    """logits [n][E] = bf16(LN(dvec + r)) . w^T without writing q (d in 1024, 2048, 4096)."""
    n, d = r.shape
    E = w.shape[0]
    logits = _empty((n, E), torch.float32, r) if logits is None else logits
    _call("route_qgate", _dev(r, _bf16(r), "r"), _dev(dvec, torch.float32, "dvec", d),
          _opt(gamma, torch.float32, "gamma", d), _opt(beta, torch.float32, "beta", d), n, d,
          float(eps), _dev(w, _bf16(w), "w", E * d), E, _dev(logits, torch.float32, "logits", n * E),
          _stream(stream))
    return logits


def route_qgate_topk(r, dvec, w, K, gamma=None, beta=None, eps=1e-5, idx=None, logits=None,
                     truth=None, hits=None, stream=None):
    """idx [n][K]: the top-K columns of bf16(LN(dvec + r)) . w^T per row (route_topk's
    order); logits [n][E] written too when given. With truth [n][K] and hits (int64 [1],
    accumulated) the kernel also counts the picks found among the true experts, as
    hit_count would. d in 1024, 2048, 4096; E <= 256."""
    n, d = r.shape
    E = w.shape[0]
    idx = _empty((n, K), torch.int32, r) if idx is None else idx
    if (truth is None) != (hits is None):
        raise ValueError("truth and hits go together")
    _call("route_qgate_topk", _dev(r, _bf16(r), "r"), _dev(dvec, torch.float32, "dvec", d),
          _opt(gamma, torch.float32, "gamma", d), _opt(beta, torch.float32, "beta", d), n, d,
          float(eps), _dev(w, _bf16(w), "w", E * d), E, K,
          _opt(logits, torch.float32, "logits", n * E), _dev(idx, torch.int32, "idx", n * K),
          _opt(truth, torch.int32, "truth", n * K), _opt(hits, torch.int64, "hits", 1),
          _stream(stream))
    return idx


def route_gate_packed_size(E: int, d: int) -> int:
    return int(lib().route_gate_packed_size(E, d))


def route_gate_pack(w, wp=None, stream=None):
    """w [E][d] bf16 -> its rows in route_qgate_topk_packed's fragment order
    (a flat bf16 tensor of route_gate_packed_size(E, d) bytes)."""
    E, d = w.shape
    nbytes = route_gate_packed_size(E, d)
    if nbytes == 0:
        raise ValueError(f"route_gate_pack: E={E}, d={d} not taken (d % 32 != 0)")
    wp = _empty((nbytes // 2,), _bf16(w), w) if wp is None else wp
    _call("route_gate_pack", _dev(w, _bf16(w), "w", E * d), E, d,
          _dev(wp, _bf16(w), "wp", nbytes // 2), _stream(stream))
    return wp


def route_est_out_topk_packed(h, w2p, b2, E, K, logits=None, idx=None, truth=None, hits=None,
                              stream=None):
    """The estimator's output layer h . w2^T + b2 with its top-K (and the hit
    count against truth) in one kernel; w2p from route_gate_pack(w2).
    Returns idx."""
    n, hd = h.shape
    idx = _empty((n, K), torch.int32, h) if idx is None else idx
    _call("route_est_out_topk_packed", _dev(h, _bf16(h), "h"), n, hd, _dev(w2p, _bf16(w2p), "w2p"),
          _opt(b2, torch.float32, "b2", E), E, K, _opt(logits, torch.float32, "logits", n * E),
          _dev(idx, torch.int32, "idx", n * K), _opt(truth, torch.int32, "truth", n * K),
          _opt(hits, torch.int64, "hits", 1), _stream(stream))
    return idx


def route_qest_hidden_packed(r, dvec, w1p, b1, hd, gamma=None, beta=None, eps=1e-5, h=None,
                             stream=None):
    """q_l and the estimator's hidden layer in one kernel: r [n][d] bf16 ->
    h = GELU(q_l W1^T + b1) [n][hd] bf16, W1 packed by route_gate_pack."""
    n, d = r.shape
    bt = _bf16(r)
    h = _empty((n, hd), bt, r) if h is None else h
    _call("route_qest_hidden_packed", _dev(r, bt, "r"), _dev(dvec, torch.float32, "dvec", d),
          _opt(gamma, torch.float32, "gamma", d), _opt(beta, torch.float32, "beta", d), n, d, eps,
          _dev(w1p, _bf16(w1p), "w1p", route_gate_packed_size(hd, d) // 2),
          _dev(b1, torch.float32, "b1", hd), hd, _dev(h, bt, "h", n * hd), _stream(stream))
    return h


def route_qest_topk_packed(r, dvec, w1p, b1, hd, w2p, b2, E, K, gamma=None, beta=None, eps=1e-5,
                           idx=None, logits=None, truth=None, hits=None, stream=None):
    """The estimator predictor of one layer in one kernel: q_l, h = GELU(q_l
    W1^T + b1) (bf16), h . W2^T + b2, its top-K and the hit count, with W1
    and W2 packed by route_gate_pack. Returns idx."""
    n, d = r.shape
    bt = _bf16(r)
    idx = _empty((n, K), torch.int32, r) if idx is None else idx
    if (truth is None) != (hits is None):
        raise ValueError("truth and hits go together")
    _call("route_qest_topk_packed", _dev(r, bt, "r"), _dev(dvec, torch.float32, "dvec", d),
          _opt(gamma, torch.float32, "gamma", d), _opt(beta, torch.float32, "beta", d), n, d, eps,
          _dev(w1p, _bf16(w1p), "w1p", route_gate_packed_size(hd, d) // 2),
          _dev(b1, torch.float32, "b1", hd), hd,
          _dev(w2p, _bf16(w2p), "w2p", route_gate_packed_size(E, hd) // 2),
          _opt(b2, torch.float32, "b2", E), E, K, _opt(logits, torch.float32, "logits", n * E),
          _dev(idx, torch.int32, "idx", n * K), _opt(truth, torch.int32, "truth", n * K),
          _opt(hits, torch.int64, "hits", 1), _stream(stream))
    return idx


def route_qgate_topk_packed(r, dvec, wp, E, K, gamma=None, beta=None, eps=1e-5, idx=None,
                            logits=None, truth=None, hits=None, stream=None):
    """route_qgate_topk with the router packed by route_gate_pack (the same
    results, bit for bit)."""
    n, d = r.shape
    idx = _empty((n, K), torch.int32, r) if idx is None else idx
    if (truth is None) != (hits is None):
        raise ValueError("truth and hits go together")
    _call("route_qgate_topk_packed", _dev(r, _bf16(r), "r"), _dev(dvec, torch.float32, "dvec", d),
          _opt(gamma, torch.float32, "gamma", d), _opt(beta, torch.float32, "beta", d), n, d,
          float(eps), _dev(wp, _bf16(wp), "wp", route_gate_packed_size(E, d) // 2), E, K,
          _opt(logits, torch.float32, "logits", n * E), _dev(idx, torch.int32, "idx", n * K),
          _opt(truth, torch.int32, "truth", n * K), _opt(hits, torch.int64, "hits", 1),
          _stream(stream))
    return idx


def route_estimator_workspace_size(n: int, hd: int) -> int:
    return int(lib().route_estimator_workspace_size(n, hd))


def route_estimator(q, w1, b1, w2, b2, logits=None, ws=None, stream=None):
    n, d = q.shape
    hd = w1.shape[0]
    E = w2.shape[0]
    logits = _empty((n, E), torch.float32, q) if logits is None else logits
    need = route_estimator_workspace_size(n, hd)
    ws = _empty((max(need, 16),), torch.uint8, q) if ws is None else ws
    _call("route_estimator", _dev(q, _bf16(q), "q"), n, d, _dev(w1, _bf16(w1), "w1", hd * d),
          _dev(b1, torch.float32, "b1", hd), hd, _dev(w2, _bf16(w2), "w2", E * hd),
          _dev(b2, torch.float32, "b2", E), E, _dev(logits, torch.float32, "logits", n * E),
          _dev(ws, torch.uint8, "ws"), ws.numel(), _stream(stream))
    return logits


def hit_count(pred, truth, hits, stream=None):
    n, K = pred.shape
    _call("hit_count", _dev(pred, torch.int32, "pred"), _dev(truth, torch.int32, "truth", n * K),
          n, K, _dev(hits, torch.int64, "hits", 1), _stream(stream))
    return hits


# ------------------------------------------------------------ s-EG placement

def eg_profile(tok, idx, row_of_id, counts, freq, err=None, stream=None):
    """counts [U][E] += activations of tok[n] routed to idx[n][K]; freq [U] += occurrences."""
    n, K = idx.shape
    U, E = counts.shape
    _call("eg_profile", _dev(tok, torch.int32, "tok", n), _dev(idx, torch.int32, "idx"), n, K,
          _dev(row_of_id, torch.int32, "row_of_id"), row_of_id.numel(), U, E,
          _dev(counts, torch.int32, "counts"), _dev(freq, torch.int32, "freq", U),
          _opt(err, torch.int32, "err", 1), _stream(stream))
    return counts, freq


def eg_init(P, best_J, stream=None):
    E, G = P.shape
    _call("eg_init", _dev(P, torch.float64, "P"), E, G, _dev(best_J, torch.float64, "best_J", 1),
          _stream(stream))
    return P, best_J


def eg_sample(P, B, seed, it, place=None, stream=None):
    E, G = P.shape
    place = _empty((B, E), torch.uint8, P) if place is None else place
    _call("eg_sample", _dev(P, torch.float64, "P"), E, G, B, int(seed) & ((1 << 64) - 1), it,
          _dev(place, torch.uint8, "place", B * E), _stream(stream))
    return place


def eg_score_workspace_size(U: int, E: int, G: int, B: int) -> int:
    return int(lib().eg_score_workspace_size(U, E, G, B))


def eg_score(counts, freq, place, G, local=None, load=None, ws=None, err=None, stream=None):
    """local [B] and load [B][G] (int64) of placements place [B][E] against a profile."""
    U, E = counts.shape
    B = place.shape[0]
    local = _empty((B,), torch.int64, place) if local is None else local
    load = _empty((B, G), torch.int64, place) if load is None else load
    need = eg_score_workspace_size(U, E, G, B)
    ws = _empty((max(need, 16),), torch.uint8, place) if ws is None else ws
    _call("eg_score", _dev(counts, torch.int32, "counts"), _dev(freq, torch.int32, "freq", U),
          U, E, G, _dev(place, torch.uint8, "place", B * E), B,
          _dev(local, torch.int64, "local", B), _dev(load, torch.int64, "load", B * G),
          _dev(ws, torch.uint8, "ws"), ws.numel(), _opt(err, torch.int32, "err", 1),
          _stream(stream))
    return local, load


def eg_update(local, load, place, total, tokens, theta, n_elite, alpha, P, best_J, best_place,
              J=None, stream=None):
    B, E = place.shape
    G = P.shape[1]
    _call("eg_update", _dev(local, torch.int64, "local", B), _dev(load, torch.int64, "load", B * G),
          _dev(place, torch.uint8, "place"), B, E, G, int(total), int(tokens), float(theta),
          int(n_elite), float(alpha), _dev(P, torch.float64, "P", E * G),
          _dev(best_J, torch.float64, "best_J", 1), _dev(best_place, torch.uint8, "best_place", E),
          _opt(J, torch.float64, "J", B), _stream(stream))
    return P, best_J, best_place


# ------------------------------------------------------------- estimator fit

def route_est_hidden(q, w1, b1, h=None, stream=None):
    """The estimator's hidden layer h [n][hd] = GELU(q W1^T + b1) (bf16)."""
    n, d = q.shape
    hd = w1.shape[0]
    h = _empty((n, hd), _bf16(q), q) if h is None else h
    _call("route_est_hidden", _dev(q, _bf16(q), "q"), n, d, _dev(w1, _bf16(w1), "w1", hd * d),
          _dev(b1, torch.float32, "b1", hd), hd, _dev(h, _bf16(h), "h", n * hd), _stream(stream))
    return h


def est_fit_gram_workspace_size(n: int, hd: int, E: int) -> int:
    return int(lib().est_fit_gram_workspace_size(n, hd, E))


def est_fit_gram(h, y, gram=None, rhs=None, ws=None, stream=None):
    """gram [hd+1][hd+1] = H'^T H', rhs [hd+1][E] = H'^T Y (float64)."""
    n, hd = h.shape
    E = y.shape[1]
    gram = _empty((hd + 1, hd + 1), torch.float64, h) if gram is None else gram
    rhs = _empty((hd + 1, E), torch.float64, h) if rhs is None else rhs
    need = est_fit_gram_workspace_size(n, hd, E)
    ws = _empty((max(need, 16),), torch.uint8, h) if ws is None else ws
    _call("est_fit_gram", _dev(h, _bf16(h), "h"), _dev(y, torch.float32, "y", n * E), n, hd, E,
          _dev(gram, torch.float64, "gram", (hd + 1) ** 2), _dev(rhs, torch.float64, "rhs", (hd + 1) * E),
          _dev(ws, torch.uint8, "ws"), ws.numel(), _stream(stream))
    return gram, rhs


def est_fit_solve(gram, rhs, ridge, info=None, stream=None):
    """In place: gram -> its Cholesky factor (after + lambda I), rhs -> W'."""
    m = gram.shape[0]
    E = rhs.shape[1]
    _call("est_fit_solve", _dev(gram, torch.float64, "gram", m * m),
          _dev(rhs, torch.float64, "rhs", m * E), m, E, float(ridge),
          _opt(info, torch.int32, "info", 1), _stream(stream))
    return rhs


def est_fit_weights(wsol, w2=None, b2=None, stream=None):
    """(w2 bf16 [E][hd], b2 float32 [E]) from W' [hd+1][E]."""
    m, E = wsol.shape
    hd = m - 1
    w2 = _empty((E, hd), torch.bfloat16, wsol) if w2 is None else w2
    b2 = _empty((E,), torch.float32, wsol) if b2 is None else b2
    _call("est_fit_weights", _dev(wsol, torch.float64, "wsol", m * E), hd, E,
          _dev(w2, _bf16(w2), "w2", E * hd), _dev(b2, torch.float32, "b2", E), _stream(stream))
    return w2, b2


# ------------------------------------------------- speculative expert prefetch

def prefetch_plan(pred, E, C, lst=None, nlist=None, err=None, stream=None):
    """list [C] int32: the distinct experts of pred [n][K] by pick count (ties to the
    lower index), -1 padded; nlist [1] int32: how many are listed."""
    n, K = pred.shape
    dev = pred.device
    lst = torch.empty(C, dtype=torch.int32, device=dev) if lst is None else lst
    nlist = torch.empty(1, dtype=torch.int32, device=dev) if nlist is None else nlist
    _call("prefetch_plan", _dev(pred, torch.int32, "pred"), n, K, E, C,
          _dev(lst, torch.int32, "list", C), _dev(nlist, torch.int32, "nlist", 1),
          _opt(err, torch.int32, "err", 1), _stream(stream))
    return lst, nlist


def prefetch_copy(bank, lst, slots, err=None, stream=None):
    """slots [C][B] uint8 <- bank [E][B] rows named by lst [C] (-1: left as is). bank may
    be a pinned host tensor (read by the GPU over PCIe) or a device tensor."""
    if not isinstance(bank, torch.Tensor) or bank.dtype != torch.uint8 or bank.dim() != 2:
        raise TypeError("bank must be a 2-D uint8 tensor [E][expert_bytes]")
    if not bank.is_contiguous():
        raise ValueError("bank must be contiguous")
    if bank.device.type != "cuda" and not bank.is_pinned():
        raise ValueError("bank must be a GPU tensor or pinned host memory")
    E, B = bank.shape
    C = lst.numel()
    _call("prefetch_copy", bank.data_ptr(), E, B, _dev(lst, torch.int32, "list"), C,
          _dev(slots, torch.uint8, "slots", C * B), _opt(err, torch.int32, "err", 1),
          _stream(stream))
    return slots


def prefetch_issue(bank, lst, slots, stream=None):
    """DMA copies (hipMemcpyAsync on ``stream``) of the bank [E][B] rows named by the
    HOST int32 list ``lst`` [C] (-1: skipped) into slots [C][B]; runs of consecutive
    experts go as one transfer. bank: pinned host or device uint8 tensor."""
    if not isinstance(bank, torch.Tensor) or bank.dtype != torch.uint8 or bank.dim() != 2:
        raise TypeError("bank must be a 2-D uint8 tensor [E][expert_bytes]")
    if not bank.is_contiguous():
        raise ValueError("bank must be contiguous")
    if bank.device.type != "cuda" and not bank.is_pinned():
        raise ValueError("bank must be a GPU tensor or pinned host memory")
    if not isinstance(lst, torch.Tensor) or lst.device.type != "cpu" or lst.dtype != torch.int32 \
            or not lst.is_contiguous():
        raise TypeError("lst must be a contiguous int32 host tensor")
    E, B = bank.shape
    C = lst.numel()
    _call("prefetch_issue", bank.data_ptr(), E, B, lst.data_ptr(), C,
          _dev(slots, torch.uint8, "slots", C * B), _stream(stream))
    return slots


def prefetch_coverage(truth, lst, E, covered, miss=None, nmiss=None, err=None, stream=None):
    """covered [1] += true picks whose expert is listed; miss [E]: the true experts
    listed nowhere, in index order, -1 padded; nmiss [1]: their number."""
    n, K = truth.shape
    dev = truth.device
    miss = torch.empty(E, dtype=torch.int32, device=dev) if miss is None else miss
    nmiss = torch.empty(1, dtype=torch.int32, device=dev) if nmiss is None else nmiss
    _call("prefetch_coverage", _dev(truth, torch.int32, "truth"), n, K, E,
          _dev(lst, torch.int32, "list"), lst.numel(), _dev(covered, torch.int64, "covered", 1),
          _dev(miss, torch.int32, "miss", E), _dev(nmiss, torch.int32, "nmiss", 1),
          _opt(err, torch.int32, "err", 1), _stream(stream))
    return miss, nmiss

