"""Comparison of the GPU path with the CPU oracle.

Rules (tolerances are relative, per row, L2):
  * selection: for each (token, head) the relative gap between the k-th and
    (k+1)-th largest flat scores (oracle, float64) is
        gap = (s_k - s_k1) / max(|s_k|, |s_k1|, 1e-30).
    Where gap > 1e-4 the GPU's index SET must equal the oracle's exactly.
    Otherwise (a near-tie, where several k-sets are correct top-k sets up to
    rounding) the GPU set must hold k distinct slots, each with oracle score
    >= s_k - 1e-4 * max(|s_k|, |s_k1|).
  * everything else is compared with the oracle recomputed on the GPU's own
    selection, so a legitimate near-tie choice is judged on its own terms:
    weights element-wise (absolute); y / dq / dkeys / dvalues per row,
    ||gpu - oracle|| / max(||oracle||, 1e-3 * rms row norm) <= tol, AND
    element by element, |gpu - oracle| <= tol * (|oracle| + rms of the row);
    y also element by element within the float32 summation bound plus (bf16)
    half a bfloat16 spacing -- what the arithmetic itself allows.
  * value-gradient rows no pick selected must be exactly zero.
"""
from __future__ import annotations

import numpy as np

GAP = 1e-4
TOL = {"fp32": 1e-4, "bf16": 2e-2}


def rel_gap(kth: np.ndarray, kth1: np.ndarray) -> np.ndarray:
    with np.errstate(invalid="ignore"):
        den = np.maximum(np.maximum(np.abs(kth), np.abs(kth1)), 1e-30)
        g = (kth - kth1) / den
    return np.where(np.isinf(kth1), np.inf, g)


def check_selection(gpu_idx: np.ndarray, ref: dict, given: dict, n: int) -> dict:
    """gpu_idx [T,H,k]; ref = oracle.forward(); given = oracle.forward_given_idx(gpu_idx)."""
    T, H, k = gpu_idx.shape
    gap = rel_gap(ref["kth"], ref["kth1"])
    strict = gap > GAP
    g_sorted = np.sort(gpu_idx, axis=2)
    o_sorted = np.sort(ref["idx"], axis=2)
    same = np.all(g_sorted == o_sorted, axis=2)
    bad_strict = strict & ~same
    assert not bad_strict.any(), (
        f"{bad_strict.sum()} (token, head) rows with gap > {GAP} select a different set; "
        f"first at {np.argwhere(bad_strict)[0].tolist()}")
    assert np.all((gpu_idx >= 0) & (gpu_idx < n * n)), "slot out of range"
    distinct = np.all(np.diff(g_sorted, axis=2) != 0, axis=2)
    assert distinct.all(), "a selection repeats a slot"
    floor = ref["kth"] - GAP * np.maximum(np.abs(ref["kth"]), np.abs(ref["kth1"]))
    ok_scores = np.all(given["scores"] >= floor[:, :, None] - 1e-12, axis=2)
    assert np.all(ok_scores | strict), "a near-tie row selected a slot scoring below the k-th"
    return dict(rows=T * H, exempt=int((~strict).sum()), exempt_differs=int((~strict & ~same).sum()))


def row_rel_err(got: np.ndarray, want: np.ndarray, floor: float = 1e-3,
                abs_floor: float = 0.0) -> np.ndarray:
    """Per-row ||got - want|| / max(||want||, floor * rms row norm of want, abs_floor).

    abs_floor is for tensors whose exact value is (nearly) all zero, where the
    rms of the reference is itself rounding noise: the caller passes 1e-3 of
    the size of one term of the sums that make a row."""
    got = got.reshape(got.shape[0], -1).astype(np.float64)
    want = want.reshape(want.shape[0], -1).astype(np.float64)
    norms = np.linalg.norm(want, axis=1)
    rms = np.sqrt(np.mean(norms ** 2)) if norms.size else 0.0
    den = np.maximum(np.maximum(norms, floor * rms), abs_floor) + 1e-300
    return np.linalg.norm(got - want, axis=1) / den


def elem_rel_err(got: np.ndarray, want: np.ndarray, floor: float = 1e-3,
                 abs_floor: float = 0.0) -> np.ndarray:
    """Per element |got - want| / (|want| + rms of want's row), rows = first
    axis.  The row term is floored like row_rel_err's denominator, scaled to
    one element: at floor * (rms row norm of the tensor) / sqrt(row length)
    and at abs_floor / sqrt(row length)."""
    got = got.reshape(got.shape[0], -1).astype(np.float64)
    want = want.reshape(want.shape[0], -1).astype(np.float64)
    if want.size == 0:
        return np.zeros(want.shape)
    ncol = want.shape[1]
    norms = np.linalg.norm(want, axis=1, keepdims=True)
    tensor_rms = np.sqrt(np.mean(norms ** 2))
    row = np.maximum(np.maximum(norms, floor * tensor_rms), abs_floor) / np.sqrt(ncol)
    return np.abs(got - want) / (np.abs(want) + row + 1e-300)


def assert_elems_close(name: str, got, want, tol: float, floor: float = 1e-3,
                       abs_floor: float = 0.0) -> float:
    """Element by element: |g - o| <= tol * (|o| + rms of the row)."""
    err = elem_rel_err(np.asarray(got), np.asarray(want), floor, abs_floor)
    worst = float(err.max()) if err.size else 0.0
    if err.size and worst > tol:
        at = np.unravel_index(int(err.argmax()), err.shape)
        raise AssertionError(f"{name}: worst element error {worst:.3e} > {tol:.1e} at (row, col) "
                             f"{tuple(int(x) for x in at)}")
    return worst


def bf16_ulp(x: np.ndarray) -> np.ndarray:
    """Spacing of bfloat16 numbers (8 significant bits) at |x|: 2^(e - 8) for
    |x| in [2^(e-1), 2^e); the subnormal spacing below the normal range."""
    m, e = np.frexp(np.abs(x))
    return np.ldexp(1.0, np.maximum(e, -125) - 8)


def assert_y_bound(name: str, got, want, bound, storage: str) -> float:
    """y element by element against what the arithmetic allows: the float32
    sums may differ from the exact value by at most `bound` (the summation
    bound, see gpu_util.y_sum_bound), and bfloat16 storage adds one rounding
    to nearest, at most half a spacing at the stored magnitude.  Returns the
    worst ratio of the error to the allowance."""
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    allow = bound + (0.5 * bf16_ulp(np.abs(want) + bound) if storage == "bf16" else 0.0)
    ratio = np.abs(got - want) / (allow + 1e-300)
    worst = float(ratio.max()) if ratio.size else 0.0
    if ratio.size and worst > 1.0:
        at = np.unravel_index(int(ratio.argmax()), ratio.shape)
        raise AssertionError(f"{name}: element {tuple(int(x) for x in at)} off by "
                             f"{abs(got[at] - want[at]):.3e}, allowed {allow[at]:.3e} "
                             f"(float32 sums + {storage} rounding)")
    return worst


def assert_rows_close(name: str, got, want, tol: float, floor: float = 1e-3,
                      abs_floor: float = 0.0) -> float:
    err = row_rel_err(np.asarray(got), np.asarray(want), floor, abs_floor)
    worst = float(err.max()) if err.size else 0.0
    assert worst <= tol, f"{name}: worst row relative error {worst:.3e} > {tol:.1e} (row {int(err.argmax())})"
    return worst
