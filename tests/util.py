"""Helpers shared by the tests: moving workload arrays to the device and the
parity metrics. Holds none of the layer's arithmetic."""
from __future__ import annotations

import numpy as np
import torch

# Tolerances of the parity gate: fp32 results within a max relative error of
# 1e-5, bf16 results (fp32 accumulation) within 2e-2 relative to the RMS of
# the reference output.
TOL_F32 = 1e-5
TOL_BF16 = 2e-2


def to_torch(a: np.ndarray, device="cuda"):
    """numpy fp32 / bf16-bits (uint16) / int32 array -> device tensor."""
    if a is None:
        return None
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def to_numpy(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def widen(a: np.ndarray) -> np.ndarray:
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def err_f32(got, ref) -> float:
    """max_i |got_i - ref_i| / max(|ref_i|, rms(ref))."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    rms = float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0
    den = np.maximum(np.abs(ref), rms if rms > 0 else 1.0)
    return float(np.max(np.abs(got - ref) / den)) if ref.size else 0.0


def err_bf16(got, ref) -> float:
    """max_i |got_i - ref_i| / rms(ref)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    if not ref.size:
        return 0.0
    rms = float(np.sqrt(np.mean(ref * ref)))
    return float(np.max(np.abs(got - ref)) / (rms if rms > 0 else 1.0))


def check_float(got, ref, dtype: str, what: str):
    """Parity gate of one float output; bf16 bit patterns (uint16) are widened
    to their values first."""
    got = widen(got) if isinstance(got, np.ndarray) and got.dtype == np.uint16 else got
    if dtype == "f32":
        e = err_f32(got, ref)
        assert e <= TOL_F32, f"{what}: max rel err {e:.3e} > {TOL_F32}"
    else:
        e = err_bf16(got, ref)
        assert e <= TOL_BF16, f"{what}: max err / rms {e:.3e} > {TOL_BF16}"
    return e


U_BF16 = 2.0 ** -8   # unit roundoff of bf16 (8 significant bits, round to nearest)


def check_bf16_stored(got, ref, what: str):
    """Parity gate of an output the method stores in bf16 (a partial sum on its
    way to the reduce-scatter). The stored value is the computed one rounded
    once more, which moves it by at most U_BF16 of its own magnitude; that
    rounding is taken off each element's error before the usual bf16 bar:
    max_i (|got_i - ref_i| - U*|ref_i|)+ / (1 + U) <= TOL_BF16 * rms(ref)."""
    got = widen(got) if got.dtype == np.uint16 else np.asarray(got, np.float64)
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    if not ref.size:
        return 0.0
    rms = float(np.sqrt(np.mean(ref * ref)))
    excess = np.maximum(np.abs(got - ref) - U_BF16 * np.abs(ref), 0.0) / (1 + U_BF16)
    e = float(excess.max()) / max(rms, 1e-30)
    assert e <= TOL_BF16, f"{what}: max (err - rounding) / rms {e:.3e} > {TOL_BF16}"
    return e


GRAD_L2_BF16 = 2e-2     # backward, bf16 data: ||got - ref||_2 / ||ref||_2
GRAD_FLIP_ULPS = 2      # backward, bf16 data: rounding flips allowed per element, in ulps


def check_grad(got, ref, dtype: str, what: str):
    """Parity gate of one gradient of the backward. fp32 data: the forward's
    max relative error 1e-5. bf16 data: ``ref`` is the oracle's chain with
    every value rounded to bf16 at the storage points where training hands it
    from one kernel to the next, all sums exact. Norm-wise, the relative L2
    error is at most 2e-2; element-wise, the forward's bar applies,
    max_i (|got_i - ref_i| - 2 ulp_i)+ / rms(ref) <= 2e-2, with 2 ulp_i =
    4 U_BF16 |ref_i| of room for rounding flips: a value stored in bf16 on
    both sides differs by one ulp where the GPU's fp32 value and the
    oracle's exact one fall on opposite sides of a rounding boundary, and a
    value formed from stored inputs moves by about one ulp more where one of
    them flipped. Returns the relative L2 error."""
    got = widen(got) if isinstance(got, np.ndarray) and got.dtype == np.uint16 else got
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    if dtype == "f32":
        e = err_f32(got, ref)
        assert e <= TOL_F32, f"{what}: max rel err {e:.3e} > {TOL_F32}"
        return e
    if not ref.size:
        return 0.0
    diff = np.abs(got - ref)
    l2 = float(np.sqrt(np.sum(diff * diff) / max(np.sum(ref * ref), 1e-300)))
    assert l2 <= GRAD_L2_BF16, f"{what}: relative L2 error {l2:.3e} > {GRAD_L2_BF16}"
    excess = np.maximum(diff - GRAD_FLIP_ULPS * 2 * U_BF16 * np.abs(ref), 0.0)
    rms = float(np.sqrt(np.mean(ref * ref)))
    mx = float(excess.max()) / max(rms, 1e-300)
    assert mx <= TOL_BF16, \
        f"{what}: max err beyond {GRAD_FLIP_ULPS} ulps / rms {mx:.3e} > {TOL_BF16}"
    return l2


def _rms(ref: np.ndarray, chunk: int) -> float:
    """RMS of a large float array, accumulated in float64 over row chunks."""
    n = ref.shape[0]
    tot = 0.0
    for r0 in range(0, n, chunk):
        blk = np.asarray(ref[r0:r0 + chunk], np.float64)
        tot += float(np.sum(blk * blk))
    return float(np.sqrt(tot / max(ref.size, 1)))


def _host_rows(got, r0: int, r1: int) -> np.ndarray:
    """Rows [r0, r1) of a device tensor or host array, widened to float64."""
    if isinstance(got, torch.Tensor):
        got = to_numpy(got[r0:r1])
    else:
        got = got[r0:r1]
    return widen(got) if got.dtype == np.uint16 else np.asarray(got, np.float64)


def check_rows(got, ref: np.ndarray, dtype: str, what: str, allowance=None,
               chunk: int = 4096) -> float:
    """Parity gate of a large 2-D float output, compared element by element in
    row chunks (bounded host memory): ``got`` is a device tensor (or host
    array) whose first len(ref) rows are compared with ``ref`` (float64).
    fp32: max_i |d_i| / max(|ref_i|, rms(ref)) <= TOL_F32; bf16:
    max_i |d_i| / rms(ref) <= TOL_BF16. ``allowance`` (bf16 only): a function
    of (r0, r1, ref block) giving the per-element storage-rounding bound that
    is taken off each error first (see check_bf16_stored)."""
    n = ref.shape[0]
    if n == 0:
        return 0.0
    rms = _rms(ref, chunk)
    worst = 0.0
    for r0 in range(0, n, chunk):
        r1 = min(n, r0 + chunk)
        g = _host_rows(got, r0, r1)
        rb = np.asarray(ref[r0:r1], np.float64)
        diff = np.abs(g - rb)
        if dtype == "f32":
            e = float(np.max(diff / np.maximum(np.abs(rb), rms if rms > 0 else 1.0)))
        else:
            if allowance is not None:
                diff = np.maximum(diff - allowance(r0, r1, rb), 0.0) / (1 + U_BF16)
            e = float(diff.max()) / (rms if rms > 0 else 1.0)
        worst = max(worst, e)
    tol = TOL_F32 if dtype == "f32" else TOL_BF16
    assert worst <= tol, f"{what}: error {worst:.3e} > {tol} ({dtype} rule)"
    return worst


def rel_l2(got, ref: np.ndarray, chunk: int = 4096) -> float:
    """||got - ref||_2 / ||ref||_2 over the first len(ref) rows, in row chunks."""
    num = den = 0.0
    for r0 in range(0, ref.shape[0], chunk):
        r1 = min(ref.shape[0], r0 + chunk)
        g = _host_rows(got, r0, r1)
        rb = np.asarray(ref[r0:r1], np.float64)
        num += float(np.sum((g - rb) ** 2))
        den += float(np.sum(rb * rb))
    return float(np.sqrt(num / max(den, 1e-300)))


def stored_bf16_allowance(r0, r1, rb):
    """Storage rounding of an output stored in bf16: at most U_BF16 of the
    element's magnitude (twice the round-to-nearest bound, for the
    difference between the computed and the exact value)."""
    return U_BF16 * np.abs(rb)


def assert_rows_equal(got, ref: np.ndarray, what: str, chunk: int = 8192):
    """Bitwise equality of a device tensor's first len(ref) rows with ``ref``,
    in row chunks."""
    n = ref.shape[0]
    for r0 in range(0, n, chunk):
        r1 = min(n, r0 + chunk)
        g = to_numpy(got[r0:r1]) if isinstance(got, torch.Tensor) else got[r0:r1]
        if not np.array_equal(g, ref[r0:r1]):
            bad = np.flatnonzero(np.any(g != ref[r0:r1], axis=tuple(range(1, ref.ndim))))
            raise AssertionError(f"{what}: rows differ, first at {r0 + int(bad[0])}")


def sample_rows(offsets: np.ndarray, per_expert: int, rng) -> np.ndarray:
    """First and last packed row of every non-empty expert plus random rows."""
    rows = []
    for e in range(len(offsets) - 1):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi <= lo:
            continue
        rows += [lo, hi - 1]
        if hi - lo > 2:
            rows += list(rng.integers(lo, hi, size=min(per_expert, hi - lo)))
    return np.unique(np.array(rows, np.int64))
