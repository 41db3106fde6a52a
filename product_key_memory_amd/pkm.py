"""PyTorch marshalling for the C ABI of libpkm.so.

Each function checks tensor placement and shapes, allocates the outputs and the
workspace with PyTorch's allocator, and passes raw device pointers plus the
current HIP stream to the library.  No arithmetic of the layer happens here.
"""
from __future__ import annotations

import torch

from . import _lib
from ._lib import PKMError, Problem

_DTYPES = {torch.float32: _lib.PKM_FP32, torch.bfloat16: _lib.PKM_BF16}


def pkm_status_string(code: int) -> str:
    return _lib.status_string(code)


def problem(T, H, n, k, d_k, d_v, dtype, keys_shared: bool = False) -> Problem:
    code = _DTYPES.get(dtype, dtype) if isinstance(dtype, torch.dtype) else dtype
    if isinstance(code, torch.dtype):
        raise TypeError(f"unsupported dtype {dtype}")
    if keys_shared:
        code = int(code) | _lib.PKM_KEYS_SHARED
    return Problem(int(T), int(H), int(n), int(k), int(d_k), int(d_v), int(code))


def pkm_workspace_bytes(p: Problem, backward: bool = False) -> int:
    return _lib.workspace_bytes(p, backward)


def _check(t: torch.Tensor, name: str, shape, dtype, device):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _shapes(q, keys, values):
    """Sizes, and whether the codebooks are shared by the heads: keys
    [H, 2, n, d_k/2] (one pair per head) or [2, n, d_k/2] (one pair for all)."""
    if q.dim() != 3 or keys.dim() not in (3, 4) or values.dim() != 2:
        raise ValueError("expected q [T,H,d_k], keys [H,2,n,d_k/2] or [2,n,d_k/2], "
                         "values [n*n,d_v]")
    T, H, d_k = q.shape
    shared = keys.dim() == 3
    n = keys.shape[-2]
    d_v = values.shape[1]
    if q.dtype not in _DTYPES:
        raise TypeError(f"unsupported dtype {q.dtype}")
    if q.device.type != "cuda":
        raise ValueError("tensors must be on a GPU")
    return T, H, n, d_k, d_v, shared


def _keys_shape(H, n, d_k, shared):
    return (2, n, d_k // 2) if shared else (H, 2, n, d_k // 2)


def pkm_forward(q: torch.Tensor, keys: torch.Tensor, values: torch.Tensor, k: int,
                want_scores: bool = True, out=None):
    """Forward pass.  Returns (y [T,d_v] in q.dtype, idx [T,H,k] int32,
    weights [T,H,k] float32, scores [T,H,k] float32 or None)."""
    T, H, n, d_k, d_v, shared = _shapes(q, keys, values)
    dev, dt = q.device, q.dtype
    _check(q, "q", (T, H, d_k), dt, dev)
    _check(keys, "keys", _keys_shape(H, n, d_k, shared), dt, dev)
    _check(values, "values", (n * n, d_v), dt, dev)
    p = problem(T, H, n, k, d_k, d_v, dt, shared)
    ws_bytes = pkm_workspace_bytes(p, False)
    if ws_bytes == (1 << 64) - 1:
        raise PKMError(2, "pkm_forward")
    if out is None:
        y = torch.empty((T, d_v), dtype=dt, device=dev)
        idx = torch.empty((T, H, k), dtype=torch.int32, device=dev)
        weights = torch.empty((T, H, k), dtype=torch.float32, device=dev)
        scores = torch.empty((T, H, k), dtype=torch.float32, device=dev) if want_scores else None
    else:
        y, idx, weights, scores = out
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev) if ws_bytes else None
    rc = _lib.forward(p, _ptr(q), _ptr(keys), _ptr(values), _ptr(y), _ptr(idx), _ptr(weights),
                      _ptr(scores), _ptr(ws), ws_bytes, _stream(dev))
    if rc != 0:
        raise PKMError(rc, "pkm_forward")
    return y, idx, weights, scores


def pkm_flat_forward(q: torch.Tensor, keys: torch.Tensor, values: torch.Tensor, k: int):
    """The flat-key search over all n*n implied keys (pkm_flat_forward_select),
    then the same gather as pkm_forward.  Returns (y, idx, weights, scores)
    like pkm_forward.  bf16, d_k = 512, 32 <= n <= 1024, k <= 32."""
    T, H, n, d_k, d_v, shared = _shapes(q, keys, values)
    dev, dt = q.device, q.dtype
    _check(q, "q", (T, H, d_k), dt, dev)
    _check(keys, "keys", _keys_shape(H, n, d_k, shared), dt, dev)
    _check(values, "values", (n * n, d_v), dt, dev)
    p = problem(T, H, n, k, d_k, d_v, dt, shared)
    y = torch.empty((T, d_v), dtype=dt, device=dev)
    idx = torch.empty((T, H, k), dtype=torch.int32, device=dev)
    weights = torch.empty((T, H, k), dtype=torch.float32, device=dev)
    scores = torch.empty((T, H, k), dtype=torch.float32, device=dev)
    rc = _lib.flat_forward_select(p, _ptr(q), _ptr(keys), _ptr(idx), _ptr(weights), _ptr(scores),
                                  _stream(dev))
    if rc != 0:
        raise PKMError(rc, "pkm_flat_forward_select")
    rc = _lib.forward_gather(p, _ptr(values), _ptr(idx), _ptr(weights), _ptr(y), _stream(dev))
    if rc != 0:
        raise PKMError(rc, "pkm_forward_gather")
    return y, idx, weights, scores


def pkm_backward(q: torch.Tensor, keys: torch.Tensor, values: torch.Tensor, idx: torch.Tensor,
                 weights: torch.Tensor, dy: torch.Tensor, dvalues: torch.Tensor | None = None,
                 out=None):
    """Backward pass.  Returns (dq [T,H,d_k], dkeys [H,2,n,d_k/2], dvalues [n*n,d_v]),
    all float32.  A given dvalues is ACCUMULATED into (pkm_backward); otherwise
    a new one is returned, written whole by pkm_backward_overwrite (rows no pick
    selected are 0)."""
    T, H, n, d_k, d_v, shared = _shapes(q, keys, values)
    dev, dt = q.device, q.dtype
    k = idx.shape[2]
    _check(q, "q", (T, H, d_k), dt, dev)
    _check(keys, "keys", _keys_shape(H, n, d_k, shared), dt, dev)
    _check(values, "values", (n * n, d_v), dt, dev)
    _check(idx, "idx", (T, H, k), torch.int32, dev)
    _check(weights, "weights", (T, H, k), torch.float32, dev)
    _check(dy, "dy", (T, d_v), dt, dev)
    p = problem(T, H, n, k, d_k, d_v, dt, shared)
    ws_bytes = pkm_workspace_bytes(p, True)
    if ws_bytes == (1 << 64) - 1:
        raise PKMError(2, "pkm_backward")
    accumulate = dvalues is not None
    if dvalues is None:
        dvalues = torch.empty((n * n, d_v), dtype=torch.float32, device=dev)
    else:
        _check(dvalues, "dvalues", (n * n, d_v), torch.float32, dev)
    if out is None:
        dq = torch.empty((T, H, d_k), dtype=torch.float32, device=dev)
        dkeys = torch.empty(_keys_shape(H, n, d_k, shared), dtype=torch.float32, device=dev)
    else:
        dq, dkeys = out
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev) if ws_bytes else None
    call = _lib.backward if accumulate else _lib.backward_overwrite
    rc = call(p, _ptr(q), _ptr(keys), _ptr(values), _ptr(idx), _ptr(weights), _ptr(dy), _ptr(dq),
              _ptr(dkeys), _ptr(dvalues), _ptr(ws), ws_bytes, _stream(dev))
    if rc != 0:
        raise PKMError(rc, "pkm_backward" if accumulate else "pkm_backward_overwrite")
    return dq, dkeys, dvalues


def pkm_backward_sgd(q: torch.Tensor, keys: torch.Tensor, values: torch.Tensor,
                     idx: torch.Tensor, weights: torch.Tensor, dy: torch.Tensor, lr: float,
                     out=None):
    """Backward pass with the sparse SGD step fused in: returns (dq, dkeys) as
    pkm_backward does, and updates `values` IN PLACE -- every row some pick
    selected becomes fmaf(-lr, g, w) rounded once to the storage type, g being
    the row's float32 gradient (pkm_backward's dvalues row).  No dvalues array
    is formed."""
    T, H, n, d_k, d_v, shared = _shapes(q, keys, values)
    dev, dt = q.device, q.dtype
    k = idx.shape[2]
    _check(q, "q", (T, H, d_k), dt, dev)
    _check(keys, "keys", _keys_shape(H, n, d_k, shared), dt, dev)
    _check(values, "values", (n * n, d_v), dt, dev)
    _check(idx, "idx", (T, H, k), torch.int32, dev)
    _check(weights, "weights", (T, H, k), torch.float32, dev)
    _check(dy, "dy", (T, d_v), dt, dev)
    p = problem(T, H, n, k, d_k, d_v, dt, shared)
    ws_bytes = pkm_workspace_bytes(p, 2)
    if ws_bytes == (1 << 64) - 1:
        raise PKMError(2, "pkm_backward_sgd")
    if out is None:
        dq = torch.empty((T, H, d_k), dtype=torch.float32, device=dev)
        dkeys = torch.empty(_keys_shape(H, n, d_k, shared), dtype=torch.float32, device=dev)
    else:
        dq, dkeys = out
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev) if ws_bytes else None
    rc = _lib.backward_sgd(p, _ptr(q), _ptr(keys), _ptr(values), _ptr(idx), _ptr(weights),
                           _ptr(dy), _ptr(dq), _ptr(dkeys), lr, _ptr(ws), ws_bytes, _stream(dev))
    if rc != 0:
        raise PKMError(rc, "pkm_backward_sgd")
    return dq, dkeys


def pkm_slot_sort(idx: torch.Tensor, n: int, out=None):
    """Groups the picks of idx [T,H,k] int32 by memory slot.  Returns
    (slot_start [n*n+1] int32, order [T*H*k] int32): the picks (ids
    t*H*k + h*k + r) of slot f are order[slot_start[f]:slot_start[f+1]]."""
    if idx.dim() != 3 or idx.dtype != torch.int32 or idx.device.type != "cuda":
        raise ValueError("idx must be a [T,H,k] int32 GPU tensor")
    T, H, k = idx.shape
    dev = idx.device
    _check(idx, "idx", (T, H, k), torch.int32, dev)
    # d_k / d_v / dtype do not enter the sort; any admissible values serve
    p = problem(T, H, n, k, 16, 8, torch.float32)
    ws_bytes = pkm_workspace_bytes(p, True)
    if ws_bytes == (1 << 64) - 1:
        raise PKMError(2, "pkm_slot_sort")
    if out is None:
        slot_start = torch.empty(n * n + 1, dtype=torch.int32, device=dev)
        order = torch.empty(T * H * k, dtype=torch.int32, device=dev)
    else:
        slot_start, order = out
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev) if ws_bytes else None
    rc = _lib.slot_sort(p, _ptr(idx), _ptr(slot_start), _ptr(order), _ptr(ws), ws_bytes,
                        _stream(dev))
    if rc != 0:
        raise PKMError(rc, "pkm_slot_sort")
    return slot_start, order


def _update_problem(values: torch.Tensor, n: int):
    if values.dim() != 2 or values.shape[0] != n * n or values.dtype not in _DTYPES:
        raise ValueError("values must be [n*n, d_v] float32 or bfloat16")
    # T, H, k, d_k do not enter the update; any admissible values serve
    return problem(0, 1, n, 1, 16, values.shape[1], values.dtype)


def pkm_sparse_sgd(values: torch.Tensor, dvalues: torch.Tensor, slot_start: torch.Tensor,
                   lr: float) -> torch.Tensor:
    """In place: values[f] -= lr * dvalues[f] for the slots f the batch selected
    (slot_start from pkm_slot_sort).  Returns values."""
    n = int(round((slot_start.numel() - 1) ** 0.5))
    p = _update_problem(values, n)
    dev = values.device
    _check(values, "values", values.shape, values.dtype, dev)
    _check(dvalues, "dvalues", values.shape, torch.float32, dev)
    _check(slot_start, "slot_start", (n * n + 1,), torch.int32, dev)
    rc = _lib.sparse_sgd(p, _ptr(values), _ptr(dvalues), _ptr(slot_start), lr, _stream(dev))
    if rc != 0:
        raise PKMError(rc, "pkm_sparse_sgd")
    return values


def pkm_sparse_adam(values: torch.Tensor, dvalues: torch.Tensor, slot_start: torch.Tensor,
                    m: torch.Tensor, v: torch.Tensor, step: int, lr: float,
                    beta1: float = 0.9, beta2: float = 0.999, eps: float = 1e-8) -> torch.Tensor:
    """In place Adam on the selected slots only (moments of other rows stand
    still).  m, v: float32 [n*n, d_v], zero before step 1.  Returns values."""
    n = int(round((slot_start.numel() - 1) ** 0.5))
    p = _update_problem(values, n)
    dev = values.device
    _check(values, "values", values.shape, values.dtype, dev)
    for t, name in ((dvalues, "dvalues"), (m, "m"), (v, "v")):
        _check(t, name, values.shape, torch.float32, dev)
    _check(slot_start, "slot_start", (n * n + 1,), torch.int32, dev)
    rc = _lib.sparse_adam(p, _ptr(values), _ptr(dvalues), _ptr(slot_start), _ptr(m), _ptr(v),
                          step, lr, beta1, beta2, eps, _stream(dev))
    if rc != 0:
        raise PKMError(rc, "pkm_sparse_adam")
    return values


def pkm_slot_usage(slot_start: torch.Tensor, counts: torch.Tensor | None = None):
    """counts [n*n] int64 += picks per slot of this batch (a new zeroed array
    if None).  Returns (counts, used) with used a 1-element int64 tensor: the
    slots with a non-zero count."""
    n = int(round((slot_start.numel() - 1) ** 0.5))
    dev = slot_start.device
    _check(slot_start, "slot_start", (n * n + 1,), torch.int32, dev)
    if counts is None:
        counts = torch.zeros(n * n, dtype=torch.int64, device=dev)
    _check(counts, "counts", (n * n,), torch.int64, dev)
    used = torch.empty(1, dtype=torch.int64, device=dev)
    p = problem(0, 1, n, 1, 16, 8, torch.float32)
    rc = _lib.slot_usage(p, _ptr(slot_start), _ptr(counts), _ptr(used), _stream(dev))
    if rc != 0:
        raise PKMError(rc, "pkm_slot_usage")
    return counts, used


def _query_problem(x: torch.Tensor, W: torch.Tensor) -> "_lib.QueryProblem":
    if x.dim() != 2 or W.dim() != 2 or x.shape[1] != W.shape[1]:
        raise ValueError("expected x [T, d_model] and W [d_out, d_model]")
    if x.dtype not in _DTYPES or W.dtype != x.dtype:
        raise TypeError("x and W must share a dtype, float32 or bfloat16")
    return _lib.QueryProblem(int(x.shape[0]), int(x.shape[1]), int(W.shape[0]), _DTYPES[x.dtype], 0)


def pkm_query_forward(x: torch.Tensor, W: torch.Tensor, gamma=None, beta=None, eps: float = 1e-5):
    """q = BN(x W^T) with batch statistics.  Returns (q [T, d_out] in x.dtype,
    z [T, d_out] float32, mean, rstd [d_out] float32)."""
    qp = _query_problem(x, W)
    dev = x.device
    T, D = x.shape[0], W.shape[0]
    _check(x, "x", x.shape, x.dtype, dev)
    _check(W, "W", W.shape, x.dtype, dev)
    for t, name in ((gamma, "gamma"), (beta, "beta")):
        if t is not None:
            _check(t, name, (D,), torch.float32, dev)
    q = torch.empty((T, D), dtype=x.dtype, device=dev)
    z = torch.empty((T, D), dtype=torch.float32, device=dev)
    mean = torch.empty(D, dtype=torch.float32, device=dev)
    rstd = torch.empty(D, dtype=torch.float32, device=dev)
    nb = _lib.query_workspace_bytes(qp, False)
    ws = torch.empty(max(nb, 1), dtype=torch.uint8, device=dev)
    rc = _lib.query_forward(qp, _ptr(x), _ptr(W), _ptr(gamma), _ptr(beta), eps, _ptr(q), _ptr(z),
                            _ptr(mean), _ptr(rstd), _ptr(ws), nb, _stream(dev))
    if rc != 0:
        raise PKMError(rc, "pkm_query_forward")
    return q, z, mean, rstd


def pkm_query_backward(x, W, gamma, z, mean, rstd, dq, want_affine: bool = True):
    """Returns (dx [T, d_model], dW [d_out, d_model], dgamma, dbeta), float32
    (dgamma, dbeta are None unless want_affine)."""
    qp = _query_problem(x, W)
    dev = x.device
    T, dm, D = x.shape[0], x.shape[1], W.shape[0]
    _check(z, "z", (T, D), torch.float32, dev)
    _check(dq, "dq", (T, D), torch.float32, dev)
    dx = torch.empty((T, dm), dtype=torch.float32, device=dev)
    dW = torch.empty((D, dm), dtype=torch.float32, device=dev)
    dgamma = torch.empty(D, dtype=torch.float32, device=dev) if want_affine else None
    dbeta = torch.empty(D, dtype=torch.float32, device=dev) if want_affine else None
    nb = _lib.query_workspace_bytes(qp, True)
    ws = torch.empty(max(nb, 1), dtype=torch.uint8, device=dev)
    rc = _lib.query_backward(qp, _ptr(x), _ptr(W), _ptr(gamma), _ptr(z), _ptr(mean), _ptr(rstd),
                             _ptr(dq), _ptr(dx), _ptr(dW), _ptr(dgamma), _ptr(dbeta), _ptr(ws), nb,
                             _stream(dev))
    if rc != 0:
        raise PKMError(rc, "pkm_query_backward")
    return dx, dW, dgamma, dbeta


class ProductKeyMemoryFunction(torch.autograd.Function):
    """y = PKM(q, keys, values) with the library's backward."""

    @staticmethod
    def forward(ctx, q, keys, values, k: int):
        y, idx, weights, _ = pkm_forward(q, keys, values, k, want_scores=False)
        ctx.save_for_backward(q, keys, values, idx, weights)
        return y

    @staticmethod
    def backward(ctx, dy):
        q, keys, values, idx, weights = ctx.saved_tensors
        dq, dkeys, dvalues = pkm_backward(q, keys, values, idx, weights,
                                          dy.contiguous().to(q.dtype))
        return dq.to(q.dtype), dkeys.to(keys.dtype), dvalues.to(values.dtype), None
