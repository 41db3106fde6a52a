"""fp64 CPU oracle of what follows the backward on the value table -- TEST
INFRASTRUCTURE ONLY (same rules as the rest of ``oracle/``: only tests, the
smoke check and bench.py's CPU-baseline leg use it; it imports nothing from
the GPU library).

The plain definitions, written out with numpy:

* slot usage (gptget.net summary of "Large Memory Layers with Product Keys",
  "Key Results": the share of memory slots in use): how many picks selected
  each slot, summed over batches, and how many slots were selected at all;
* sparse update (same page, "Methodology": trained end to end with sparse
  updates, only the selected slots change): SGD, w - lr * g, and Adam with
  moments advanced only for selected rows, on the rows some pick selected;
  every other row is returned unchanged.

The update is computed in float64 from the float32 (or bfloat16-widened)
inputs and rounded once to float32, then (bfloat16 storage) to bfloat16 with
round-to-nearest-even.  The GPU rounds its float32 fused result once to the
storage type; the two agree except where float64 -> float32 rounding lands
on a tie (double rounding), so tests compare within one unit in the last
place.
"""
from __future__ import annotations

import numpy as np


def touched_slots(idx_batches, n: int) -> np.ndarray:
    """Boolean [n*n]: slot selected by at least one pick of the batches."""
    mask = np.zeros(n * n, dtype=bool)
    for idx in idx_batches:
        mask[np.asarray(idx, dtype=np.int64).ravel()] = True
    return mask


def slot_usage(idx_batches, n: int):
    """(counts [n*n] int64: picks per slot over all batches, used: slots with
    a non-zero count)."""
    counts = np.zeros(n * n, dtype=np.int64)
    for idx in idx_batches:
        flat = np.asarray(idx, dtype=np.int64).ravel()
        np.add.at(counts, flat, 1)
    return counts, int(np.count_nonzero(counts))


def _round_bf16(x32: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), nearest, ties to even."""
    u = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def _widen(values: np.ndarray) -> np.ndarray:
    if values.dtype == np.uint16:
        return (values.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return values.astype(np.float64)


def _store(x64: np.ndarray, like: np.ndarray) -> np.ndarray:
    x32 = x64.astype(np.float32)
    return _round_bf16(x32) if like.dtype == np.uint16 else x32


def sparse_sgd(values: np.ndarray, dvalues: np.ndarray, touched: np.ndarray, lr: float):
    """values [R][d_v] float32 or uint16 (bf16 bits) for the rows `touched`
    (bool [R]) says were selected: w - lr * g on those rows, others as given."""
    out = values.copy()
    rows = np.nonzero(touched)[0]
    w = _widen(values[rows])
    g = dvalues[rows].astype(np.float64)
    out[rows] = _store(w - np.float64(np.float32(lr)) * g, values)
    return out


def sparse_adam(values, dvalues, touched, m, v, step: int, lr: float, beta1: float,
                beta2: float, eps: float):
    """Adam on the selected rows; returns (values, m, v), with m, v float32.
    The bias corrections c1 = 1 - beta1^step, c2 = 1 - beta2^step are taken
    in double and rounded to float32, as the boundary specifies."""
    out, mo, vo = values.copy(), m.copy(), v.copy()
    rows = np.nonzero(touched)[0]
    b1, b2 = np.float64(np.float32(beta1)), np.float64(np.float32(beta2))
    c1 = np.float64(np.float32(1.0 - np.float64(np.float32(beta1)) ** step))
    c2 = np.float64(np.float32(1.0 - np.float64(np.float32(beta2)) ** step))
    g = dvalues[rows].astype(np.float64)
    mn = b1 * m[rows].astype(np.float64) + (1.0 - b1) * g
    vn = b2 * v[rows].astype(np.float64) + (1.0 - b2) * g * g
    upd = (mn / c1) / (np.sqrt(vn / c2) + np.float64(np.float32(eps)))
    out[rows] = _store(_widen(values[rows]) - np.float64(np.float32(lr)) * upd, values)
    mo[rows] = mn.astype(np.float32)
    vo[rows] = vn.astype(np.float32)
    return out, mo, vo
