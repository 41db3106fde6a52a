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
  * dq and dkeys are compared with the oracle's backward at the weights the
    GPU backward was handed; a row (or element) whose sum cancels far below
    the size of its terms may instead lie within the float32 error bound of
    that sum (grad_sum_bound): any rounding of a term then outweighs it.
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
                abs_floor: float = 0.0, den_floor=None) -> np.ndarray:
    """Per-row ||got - want|| / max(||want||, floor * rms row norm of want, abs_floor).

    abs_floor is for tensors whose exact value is (nearly) all zero, where the
    rms of the reference is itself rounding noise: the caller passes 1e-3 of
    the size of one term of the sums that make a row.  den_floor, if given, is
    a further per-row floor of the denominator."""
    got = got.reshape(got.shape[0], -1).astype(np.float64)
    want = want.reshape(want.shape[0], -1).astype(np.float64)
    norms = np.linalg.norm(want, axis=1)
    rms = np.sqrt(np.mean(norms ** 2)) if norms.size else 0.0
    den = np.maximum(np.maximum(norms, floor * rms), abs_floor)
    if den_floor is not None:
        den = np.maximum(den, np.asarray(den_floor, np.float64).reshape(-1))
    return np.linalg.norm(got - want, axis=1) / (den + 1e-300)


def elem_rel_err(got: np.ndarray, want: np.ndarray, floor: float = 1e-3,
                 abs_floor: float = 0.0, elem_floor=None) -> np.ndarray:
    """Per element |got - want| / (|want| + rms of want's row), rows = first
    axis.  The row term is floored like row_rel_err's denominator, scaled to
    one element: at floor * (rms row norm of the tensor) / sqrt(row length)
    and at abs_floor / sqrt(row length).  elem_floor, if given (the shape of
    want), is added to each element's denominator."""
    got = got.reshape(got.shape[0], -1).astype(np.float64)
    want = want.reshape(want.shape[0], -1).astype(np.float64)
    if want.size == 0:
        return np.zeros(want.shape)
    ncol = want.shape[1]
    norms = np.linalg.norm(want, axis=1, keepdims=True)
    tensor_rms = np.sqrt(np.mean(norms ** 2))
    row = np.maximum(np.maximum(norms, floor * tensor_rms), abs_floor) / np.sqrt(ncol)
    den = np.abs(want) + row
    if elem_floor is not None:
        den = den + np.asarray(elem_floor, np.float64).reshape(want.shape)
    return np.abs(got - want) / (den + 1e-300)


def assert_elems_close(name: str, got, want, tol: float, floor: float = 1e-3,
                       abs_floor: float = 0.0, allow=None) -> float:
    """Element by element: |g - o| <= tol * (|o| + rms of the row) + allow,
    allow (the shape of want, or None) being an absolute rounding allowance
    such as gpu_util.grad_sum_bound's."""
    err = elem_rel_err(np.asarray(got), np.asarray(want), floor, abs_floor,
                       None if allow is None else np.asarray(allow) / tol)
    worst = float(err.max()) if err.size else 0.0
    if err.size and worst > tol:
        at = np.unravel_index(int(err.argmax()), err.shape)
        raise AssertionError(f"{name}: worst element error {worst:.3e} > {tol:.1e} at (row, col) "
                             f"{tuple(int(x) for x in at)}")
    return worst


def _widen(a: np.ndarray) -> np.ndarray:
    """float64 copy of float32 data or of bfloat16 bit patterns (uint16)."""
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def grad_sum_bound(q, keys, values, idx, w, dy, shared: bool = False, chunk: int = 64) -> dict:
    """Per element of dq [T][H][d_k] and dkeys ([H][2][n][d_k/2], or
    [2][n][d_k/2] summed over the heads when `shared`): how far a float32
    evaluation may lie from the exact gradients at the same weights w, in any
    order of the sums.

    Pick e of (t, h) (slot f = i n + j) has dw_e = <dy_t, values[f]> (d_v
    multiply-adds), s = sum_e' w_e' dw_e' (k more) and ds_e = w_e (dw_e - s);
    with a_e = sum_c |dy_t[c]| |values[f][c]|, every rounding up to ds_e is
    covered by m_e = |w_e| (a_e + sum_e' |w_e'| a_e').  An element of dq or
    dkeys sums r products ds_e x (x a sub-key or query element: one more
    rounding each), so the classic bound on chains of rounded operations gives
        |error| <= gamma(d_v + k + 3 + r) * sum_e m_e |x|,
    gamma(m) = m u / (1 - m u), u = 2^-24, r = k for dq and the number of
    picks of the sub-key for dkeys.  Exact-arithmetic cancellation (a token
    whose k picks share a sub-key contributes sum_e ds_e = s (1 - sum w) ~ 0)
    leaves results far below sum_e m_e |x|: only this bound holds there."""
    T, H, k = idx.shape
    n, half = keys.shape[-2], keys.shape[-1]
    d_v = values.shape[1]
    qa = np.abs(_widen(q)).reshape(T, H, 2, half)
    ka = np.abs(_widen(keys)).reshape(-1, 2, n, half)
    va, dya = np.abs(_widen(values)), np.abs(_widen(dy))
    a = np.empty((T, H, k))
    for t0 in range(0, T, chunk):
        t1 = min(T, t0 + chunk)
        rows = va[idx[t0:t1].reshape(-1)].reshape(t1 - t0, H * k, d_v)
        a[t0:t1] = np.einsum("tpc,tc->tp", rows, dya[t0:t1]).reshape(t1 - t0, H, k)
    aw = np.abs(np.asarray(w, np.float64))
    m = aw * (a + np.sum(aw * a, axis=2, keepdims=True))
    u = 2.0 ** -24

    def gamma(r):
        r = np.asarray(r, np.float64)
        return r * u / (1.0 - r * u)

    dq = np.empty((T, H, 2, half))
    dk = np.zeros((1 if shared else H, 2, n, half))
    picks = np.zeros((1 if shared else H, 2, n))
    mag = np.zeros_like(dk)
    tt = np.repeat(np.arange(T), k)
    for h in range(H):
        hk = 0 if shared else h
        for s, sub in ((0, idx[:, h] // n), (1, idx[:, h] % n)):
            M = np.zeros((T, n))             # M[t][i] = sum of m_e over t's picks of sub-key i
            np.add.at(M, (tt, sub.reshape(-1)), m[:, h].reshape(-1))
            dq[:, h, s] = gamma(d_v + 2 * k + 3) * (M @ ka[0 if shared else h, s])
            mag[hk, s] += M.T @ qa[:, h, s]
            picks[hk, s] += np.bincount(sub.reshape(-1), minlength=n)
    dk = gamma(d_v + k + 3 + picks)[..., None] * mag
    return {"dq": dq.reshape(T, H, 2 * half), "dkeys": dk[0] if shared else dk}


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
                      abs_floor: float = 0.0, allow=None) -> float:
    """Row by row: ||g - o|| <= tol * max(||o||, floors), or within the norm
    of the row of `allow` (an absolute per-element rounding allowance such as
    gpu_util.grad_sum_bound's, the shape of want; None for none)."""
    den_floor = None
    if allow is not None:
        a = np.asarray(allow, np.float64)
        den_floor = np.linalg.norm(a.reshape(a.shape[0], -1), axis=1) / tol
    err = row_rel_err(np.asarray(got), np.asarray(want), floor, abs_floor, den_floor)
    worst = float(err.max()) if err.size else 0.0
    assert worst <= tol, f"{name}: worst row relative error {worst:.3e} > {tol:.1e} (row {int(err.argmax())})"
    return worst
