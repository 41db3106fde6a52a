"""ctypes view of libpkm.so (the C ABI declared in include/pkm.h).

Loading fails loudly: there is no fallback path.  If the library has not been
built (``python -m product_key_memory_amd.build``) every entry point raises.
"""
from __future__ import annotations

import ctypes
import os

# PKM_LIB may name another build of the same library (e.g. a variant under test)
LIB_PATH = os.environ.get("PKM_LIB") or os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                                     "libpkm.so")

PKM_FP32 = 0
PKM_BF16 = 1
PKM_KEYS_SHARED = 0x100      # or-ed into Problem.dtype: one codebook pair for every head

STATUS = {
    0: "PKM_OK",
    1: "PKM_ERR_NULL",
    2: "PKM_ERR_SHAPE",
    3: "PKM_ERR_DTYPE",
    4: "PKM_ERR_WORKSPACE",
    5: "PKM_ERR_HIP",
    6: "PKM_ERR_ALIGN",
    7: "PKM_ERR_ARG",
    8: "PKM_ERR_TOO_LARGE",
}

# every symbol include/pkm.h declares
EXPORTS = ("pkm_workspace_bytes", "pkm_forward", "pkm_backward", "pkm_backward_overwrite",
           "pkm_backward_noalloc", "pkm_backward_sgd",
           "pkm_forward_select", "pkm_flat_forward_select",
           "pkm_forward_gather", "pkm_slot_sort", "pkm_backward_values", "pkm_backward_queries",
           "pkm_sparse_sgd", "pkm_sparse_adam", "pkm_slot_usage", "pkm_query_workspace_bytes",
           "pkm_query_forward", "pkm_query_backward", "pkm_status_string")


class QueryProblem(ctypes.Structure):
    """pkm_query_problem_t: int64 T, then int32 d_model, d_out, dtype, reserved (24 bytes)."""
    _fields_ = [("T", ctypes.c_int64), ("d_model", ctypes.c_int32), ("d_out", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class Problem(ctypes.Structure):
    """pkm_problem_t: int64 T, then int32 H, n, k, d_k, d_v, dtype (32 bytes)."""
    _fields_ = [("T", ctypes.c_int64), ("H", ctypes.c_int32), ("n", ctypes.c_int32),
                ("k", ctypes.c_int32), ("d_k", ctypes.c_int32), ("d_v", ctypes.c_int32),
                ("dtype", ctypes.c_int32)]


class PKMError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {status_string(code)} ({code})")


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"libpkm.so is not built at {LIB_PATH}; run `python -m product_key_memory_amd.build` "
                "(the HIP library is required: there is no CPU fallback)")
        L = ctypes.CDLL(LIB_PATH)
        P, c_size = ctypes.c_void_p, ctypes.c_size_t
        L.pkm_workspace_bytes.argtypes = [ctypes.POINTER(Problem), ctypes.c_int]
        L.pkm_workspace_bytes.restype = c_size
        L.pkm_forward.argtypes = [ctypes.POINTER(Problem), P, P, P, P, P, P, P, P, c_size, P]
        L.pkm_forward.restype = ctypes.c_int
        for name in ("pkm_backward", "pkm_backward_overwrite"):
            getattr(L, name).argtypes = [ctypes.POINTER(Problem), P, P, P, P, P, P, P, P, P, P,
                                         c_size, P]
            getattr(L, name).restype = ctypes.c_int
        L.pkm_backward_noalloc.argtypes = [ctypes.POINTER(Problem), P, P, P, P, P, P, P, P, P, P]
        L.pkm_backward_noalloc.restype = ctypes.c_int
        L.pkm_backward_sgd.argtypes = [ctypes.POINTER(Problem), P, P, P, P, P, P, P, P,
                                       ctypes.c_float, P, c_size, P]
        L.pkm_backward_sgd.restype = ctypes.c_int
        PP = ctypes.POINTER(Problem)
        L.pkm_forward_select.argtypes = [PP, P, P, P, P, P, P, c_size, P]
        L.pkm_forward_gather.argtypes = [PP, P, P, P, P, P]
        L.pkm_flat_forward_select.argtypes = [PP, P, P, P, P, P, P]
        L.pkm_slot_sort.argtypes = [PP, P, P, P, P, c_size, P]
        L.pkm_backward_values.argtypes = [PP, P, P, P, P, P, P, P, ctypes.c_int, P, P, c_size, P]
        L.pkm_backward_queries.argtypes = [PP, P, P, P, P, P, P, P, P, c_size, P]
        F, I64 = ctypes.c_float, ctypes.c_int64
        L.pkm_sparse_sgd.argtypes = [PP, P, P, P, F, P]
        L.pkm_sparse_adam.argtypes = [PP, P, P, P, P, P, I64, F, F, F, F, P]
        L.pkm_slot_usage.argtypes = [PP, P, P, P, P]
        QP = ctypes.POINTER(QueryProblem)
        L.pkm_query_workspace_bytes.argtypes = [QP, ctypes.c_int]
        L.pkm_query_workspace_bytes.restype = c_size
        L.pkm_query_forward.argtypes = [QP, P, P, P, P, F, P, P, P, P, P, c_size, P]
        L.pkm_query_backward.argtypes = [QP, P, P, P, P, P, P, P, P, P, P, P, P, c_size, P]
        for name in ("pkm_forward_select", "pkm_flat_forward_select", "pkm_forward_gather",
                     "pkm_slot_sort",
                     "pkm_backward_values", "pkm_backward_queries", "pkm_sparse_sgd",
                     "pkm_sparse_adam", "pkm_slot_usage", "pkm_query_forward",
                     "pkm_query_backward"):
            getattr(L, name).restype = ctypes.c_int
        L.pkm_status_string.argtypes = [ctypes.c_int]
        L.pkm_status_string.restype = ctypes.c_char_p
        _lib = L
    return _lib


def status_string(code: int) -> str:
    return lib().pkm_status_string(code).decode()


def workspace_bytes(p: Problem, backward) -> int:
    """backward: 0 (forward), 1 (backward and its stages), 2 (backward_sgd)."""
    return int(lib().pkm_workspace_bytes(ctypes.byref(p), int(backward)))


def forward(p: Problem, q, keys, values, y, idx, weights, scores, ws, ws_bytes, stream) -> int:
    return lib().pkm_forward(ctypes.byref(p), q, keys, values, y, idx, weights, scores, ws,
                             ws_bytes, stream)


def backward(p: Problem, q, keys, values, idx, weights, dy, dq, dkeys, dvalues, ws, ws_bytes,
             stream) -> int:
    """pkm_backward: dvalues accumulated (+=)."""
    return lib().pkm_backward(ctypes.byref(p), q, keys, values, idx, weights, dy, dq, dkeys,
                              dvalues, ws, ws_bytes, stream)


def backward_overwrite(p: Problem, q, keys, values, idx, weights, dy, dq, dkeys, dvalues, ws,
                       ws_bytes, stream) -> int:
    """pkm_backward_overwrite: dvalues overwritten (unselected rows become 0)."""
    return lib().pkm_backward_overwrite(ctypes.byref(p), q, keys, values, idx, weights, dy, dq,
                                        dkeys, dvalues, ws, ws_bytes, stream)


def backward_noalloc(p: Problem, q, keys, values, idx, weights, dy, dq, dkeys, dvalues,
                     stream) -> int:
    """pkm_backward_noalloc: pkm_backward with the library's static scratch."""
    return lib().pkm_backward_noalloc(ctypes.byref(p), q, keys, values, idx, weights, dy, dq,
                                      dkeys, dvalues, stream)


def backward_sgd(p: Problem, q, keys, values, idx, weights, dy, dq, dkeys, lr, ws, ws_bytes,
                 stream) -> int:
    return lib().pkm_backward_sgd(ctypes.byref(p), q, keys, values, idx, weights, dy, dq, dkeys,
                                  float(lr), ws, ws_bytes, stream)


def forward_select(p: Problem, q, keys, idx, weights, scores, ws, ws_bytes, stream) -> int:
    return lib().pkm_forward_select(ctypes.byref(p), q, keys, idx, weights, scores, ws, ws_bytes,
                                    stream)


def flat_forward_select(p: Problem, q, keys, idx, weights, scores, stream) -> int:
    """pkm_flat_forward_select: the flat search over all n*n implied keys."""
    return lib().pkm_flat_forward_select(ctypes.byref(p), q, keys, idx, weights, scores, stream)


def forward_gather(p: Problem, values, idx, weights, y, stream) -> int:
    return lib().pkm_forward_gather(ctypes.byref(p), values, idx, weights, y, stream)


def slot_sort(p: Problem, idx, slot_start, order, ws, ws_bytes, stream) -> int:
    return lib().pkm_slot_sort(ctypes.byref(p), idx, slot_start, order, ws, ws_bytes, stream)


def backward_values(p: Problem, values, idx, weights, dy, slot_start, order, dvalues,
                    accumulate, dw, ws, ws_bytes, stream) -> int:
    return lib().pkm_backward_values(ctypes.byref(p), values, idx, weights, dy, slot_start, order,
                                     dvalues, int(accumulate), dw, ws, ws_bytes, stream)


def backward_queries(p: Problem, q, keys, idx, weights, dw, dq, dkeys, ws, ws_bytes,
                     stream) -> int:
    return lib().pkm_backward_queries(ctypes.byref(p), q, keys, idx, weights, dw, dq, dkeys, ws,
                                      ws_bytes, stream)


def sparse_sgd(p: Problem, values, dvalues, slot_start, lr, stream) -> int:
    return lib().pkm_sparse_sgd(ctypes.byref(p), values, dvalues, slot_start, float(lr), stream)


def sparse_adam(p: Problem, values, dvalues, slot_start, m, v, step, lr, beta1, beta2, eps,
                stream) -> int:
    return lib().pkm_sparse_adam(ctypes.byref(p), values, dvalues, slot_start, m, v, int(step),
                                 float(lr), float(beta1), float(beta2), float(eps), stream)


def slot_usage(p: Problem, slot_start, counts, used, stream) -> int:
    return lib().pkm_slot_usage(ctypes.byref(p), slot_start, counts, used, stream)


def query_workspace_bytes(qp: QueryProblem, backward: bool) -> int:
    return int(lib().pkm_query_workspace_bytes(ctypes.byref(qp), int(backward)))


def query_forward(qp: QueryProblem, x, W, gamma, beta, eps, q, z, mean, rstd, ws, ws_bytes,
                  stream) -> int:
    return lib().pkm_query_forward(ctypes.byref(qp), x, W, gamma, beta, float(eps), q, z, mean,
                                   rstd, ws, ws_bytes, stream)


def query_backward(qp: QueryProblem, x, W, gamma, z, mean, rstd, dq, dx, dW, dgamma, dbeta, ws,
                   ws_bytes, stream) -> int:
    return lib().pkm_query_backward(ctypes.byref(qp), x, W, gamma, z, mean, rstd, dq, dx, dW,
                                    dgamma, dbeta, ws, ws_bytes, stream)
