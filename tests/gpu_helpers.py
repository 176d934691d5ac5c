"""Helpers for the GPU parity tests: host<->device copies and the tolerance
checks the tests assert."""
import numpy as np
import torch

from oracle.bf16 import bf16_to_f64, round_bf16

DEV = "cuda"


def dev(a: np.ndarray) -> torch.Tensor:
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def rel_err_rowfloor(got: np.ndarray, ref: np.ndarray) -> float:
    """max_ij |got - ref| / max(|ref_ij|, rms(ref_i)): elementwise relative
    error with each row's rms as the floor near zero."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    rms = np.sqrt(np.mean(ref * ref, axis=-1, keepdims=True))
    den = np.maximum(np.abs(ref), rms)
    den = np.where(den == 0, 1.0, den)
    return float(np.max(np.abs(got - ref) / den)) if got.size else 0.0


def floor_only(got, ref, tol) -> int:
    """How many elements meet |got - ref| <= tol * rms(row of ref) but not
    |got - ref| <= tol * |ref|: those the row floor alone lets through
    (reference values near zero, where a relative error has no meaning)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    diff = np.abs(got - ref)
    return int(np.count_nonzero(diff > tol * np.abs(ref)))


def assert_rel(got, ref, tol, what, max_floor_frac=None):
    """Row-floored relative error within ``tol``; prints how many elements
    pass only through the floor and, when ``max_floor_frac`` is given, bounds
    that share."""
    e = rel_err_rowfloor(got, ref)
    assert e <= tol, f"{what}: max relative error {e:.3e} > {tol:.1e}"
    nf = floor_only(got, ref, tol)
    size = max(np.size(ref), 1)
    print(f"{what}: max rel err {e:.3e}; {nf} of {np.size(ref)} elements within the row floor only")
    if max_floor_frac is not None:
        assert nf <= max_floor_frac * size, f"{what}: {nf} elements pass only through the floor"
    return e


def bf16_ulps(got_bits: np.ndarray, ref: np.ndarray) -> int:
    """Max distance in bf16 ulps between bf16 results and the nearest-even
    bf16 rounding of the float64 reference (same sign assumed away from 0)."""
    want = round_bf16(ref).astype(np.int64)
    got = np.asarray(got_bits).astype(np.int64)
    # map sign-magnitude bit patterns onto a monotone integer line
    def line(b):
        return np.where(b & 0x8000, -(b & 0x7FFF), b & 0x7FFF)
    return int(np.max(np.abs(line(got) - line(want)))) if got.size else 0


def assert_bf16(got_bits, ref, what, floor=1e-3, max_floor_frac=1e-3):
    """bf16 outputs against a float64 reference: each element within one bf16
    ulp of the reference's nearest-even rounding, or within floor * rms(row of
    the reference) where the sum cancels (near zero one bf16 ulp is smaller
    than the binary32 accumulation error). The elements that pass only
    through that floor are counted, printed and bounded: at most
    ``max_floor_frac`` of all elements. Returns the count."""
    want = round_bf16(ref).astype(np.int64)
    got = np.asarray(got_bits).astype(np.int64)
    line = lambda b: np.where(b & 0x8000, -(b & 0x7FFF), b & 0x7FFF)
    ulps = np.abs(line(got) - line(want))
    ref = np.asarray(ref, dtype=np.float64)
    rms = np.sqrt(np.mean(ref * ref, axis=-1, keepdims=True))
    near = np.abs(bf16_to_f64(got_bits) - ref) <= floor * rms
    bad = (ulps > 1) & ~near
    assert not bad.any(), f"{what}: {int(bad.sum())} elements beyond 1 ulp / {floor} rms; max ulps {int(ulps.max())}"
    nf = int(np.count_nonzero((ulps > 1) & near))
    print(f"{what}: {nf} of {ulps.size} elements beyond 1 ulp, within {floor} x row rms")
    assert nf <= max_floor_frac * max(ulps.size, 1), f"{what}: {nf} elements pass only through the floor"
    return nf


def sync():
    torch.cuda.synchronize()


def assert_dot_bound(got, ref, absref, d, what):
    """Binary32 dot products of d exact bf16 products against the float64
    ones: |got - ref| <= d * 2^-24 * sum_k |x_k w_k| (absref), the forward
    error bound of binary32 summation in any order (gamma_d with the d u
    first-order term; d u << 1 here). Unlike a relative error, this holds
    where the products cancel."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    bound = d * 2.0 ** -24 * np.asarray(absref, dtype=np.float64) * 1.001
    over = np.abs(got - ref) > bound
    assert not np.any(over), (f"{what}: {int(np.count_nonzero(over))} elements beyond the binary32 "
                              f"summation bound")
