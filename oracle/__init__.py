"""fp64 CPU oracle of the product-key memory layer -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check of ``__graft_entry__`` and the CPU-baseline
leg of ``bench.py`` may import this package.  The GPU library and its Python
binding never import it, and it imports nothing from them: it wraps
``pkm_oracle.c`` (plain C, double precision, OpenMP over tokens) through ctypes.

What each function computes, with the passages it follows, is documented in
``pkm_oracle.c``.  Arrays are numpy: float32, float64, or uint16 holding raw
bfloat16 bit patterns.  Every value is widened exactly to double inside the C
code before any arithmetic.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "pkm_oracle.c")
LIB_PATH = os.path.join(_HERE, "libpkm_oracle.so")

_I64 = ctypes.c_int64
_I32 = ctypes.c_int
_P = ctypes.c_void_p


def build(src: str = _SRC, out: str = LIB_PATH, extra_flags: tuple = ()) -> str:
    """Compile the oracle with gcc (OpenMP); returns the library path."""
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", *extra_flags,
           src, "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


class Oracle:
    """ctypes handle on one compiled copy of the oracle."""

    def __init__(self, path: str = LIB_PATH):
        if not os.path.exists(path):
            raise FileNotFoundError(f"oracle library not built: {path} (run oracle.build())")
        lib = ctypes.CDLL(path)
        lib.pkm_oracle_flat_scores.argtypes = [_I64, _I32, _I64, _I32, _I32, _I32,
                                               _P, _I32, _P, _I32, _P]
        lib.pkm_oracle_forward.argtypes = [_I64, _I32, _I32, _I32, _I32, _I32,
                                           _P, _I32, _P, _I32, _P, _I32,
                                           _P, _P, _P, _P, _P, _P, _I32]
        lib.pkm_oracle_forward_given_idx.argtypes = [_I64, _I32, _I32, _I32, _I32, _I32,
                                                     _P, _I32, _P, _I32, _P, _I32, _P,
                                                     _P, _P, _P, _I32]
        lib.pkm_oracle_backward.argtypes = [_I64, _I32, _I32, _I32, _I32, _I32,
                                            _P, _I32, _P, _I32, _P, _I32, _P, _P, _P, _I32,
                                            _P, _P, _P, _P, _P, _I32]
        lib.pkm_oracle_max_threads.argtypes = []
        lib.pkm_oracle_max_threads.restype = _I32
        self.lib = lib
        self.path = path

    # -- helpers -----------------------------------------------------------
    @staticmethod
    def _in(a: np.ndarray):
        a = np.ascontiguousarray(a)
        if a.dtype == np.float32:
            code = 0
        elif a.dtype == np.uint16:
            code = 1
        elif a.dtype == np.float64:
            code = 2
        else:
            raise TypeError(f"oracle input dtype {a.dtype} (want float32, float64 or uint16=bf16)")
        return a, a.ctypes.data_as(_P), code

    @staticmethod
    def _ptr(a):
        return None if a is None else a.ctypes.data_as(_P)

    @staticmethod
    def _shape(q, keys, values):
        T, H, d_k = q.shape
        H2, two, n, half = keys.shape
        nn, d_v = values.shape
        if H2 != H or two != 2 or half * 2 != d_k or nn != n * n:
            raise ValueError(f"inconsistent shapes q{q.shape} keys{keys.shape} values{values.shape}")
        return T, H, n, d_k, d_v

    def max_threads(self) -> int:
        return int(self.lib.pkm_oracle_max_threads())

    # -- entry points ------------------------------------------------------
    def flat_scores(self, q, keys, t: int, h: int) -> np.ndarray:
        """All n*n implied-key scores of token t, head h (slot f = i*n + j)."""
        q, qp, qd = self._in(q)
        keys, kp, kd = self._in(keys)
        T, H, d_k = q.shape
        n = keys.shape[2]
        out = np.empty(n * n, dtype=np.float64)
        rc = self.lib.pkm_oracle_flat_scores(t, h, T, H, n, d_k, qp, qd, kp, kd, self._ptr(out))
        if rc != 0:
            raise RuntimeError(f"pkm_oracle_flat_scores failed: {rc}")
        return out

    def forward(self, q, keys, values, k: int, nthreads: int = 0) -> dict:
        q, qp, qd = self._in(q)
        keys, kp, kd = self._in(keys)
        values, vp, vd = self._in(values)
        T, H, n, d_k, d_v = self._shape(q, keys, values)
        idx = np.empty((T, H, k), dtype=np.int32)
        scores = np.empty((T, H, k), dtype=np.float64)
        weights = np.empty((T, H, k), dtype=np.float64)
        y = np.empty((T, d_v), dtype=np.float64)
        kth = np.empty((T, H), dtype=np.float64)
        kth1 = np.empty((T, H), dtype=np.float64)
        rc = self.lib.pkm_oracle_forward(T, H, n, k, d_k, d_v, qp, qd, kp, kd, vp, vd,
                                         self._ptr(idx), self._ptr(scores), self._ptr(weights),
                                         self._ptr(y), self._ptr(kth), self._ptr(kth1), nthreads)
        if rc != 0:
            raise RuntimeError(f"pkm_oracle_forward failed: {rc}")
        return dict(idx=idx, scores=scores, weights=weights, y=y, kth=kth, kth1=kth1)

    def forward_given_idx(self, q, keys, values, idx, nthreads: int = 0) -> dict:
        q, qp, qd = self._in(q)
        keys, kp, kd = self._in(keys)
        values, vp, vd = self._in(values)
        T, H, n, d_k, d_v = self._shape(q, keys, values)
        idx = np.ascontiguousarray(idx, dtype=np.int32)
        k = idx.shape[2]
        scores = np.empty((T, H, k), dtype=np.float64)
        weights = np.empty((T, H, k), dtype=np.float64)
        y = np.empty((T, d_v), dtype=np.float64)
        rc = self.lib.pkm_oracle_forward_given_idx(T, H, n, k, d_k, d_v, qp, qd, kp, kd, vp, vd,
                                                   self._ptr(idx), self._ptr(scores),
                                                   self._ptr(weights), self._ptr(y), nthreads)
        if rc != 0:
            raise RuntimeError(f"pkm_oracle_forward_given_idx failed: {rc}")
        return dict(idx=idx, scores=scores, weights=weights, y=y)

    def backward(self, q, keys, values, idx, weights, dy, nthreads: int = 0,
                 want_dvalues: bool = True) -> dict:
        q, qp, qd = self._in(q)
        keys, kp, kd = self._in(keys)
        values, vp, vd = self._in(values)
        dy, dyp, dyd = self._in(dy)
        T, H, n, d_k, d_v = self._shape(q, keys, values)
        idx = np.ascontiguousarray(idx, dtype=np.int32)
        weights = np.ascontiguousarray(weights, dtype=np.float64)
        k = idx.shape[2]
        dq = np.empty((T, H, d_k), dtype=np.float64)
        dkeys = np.empty(keys.shape, dtype=np.float64)
        dvalues = np.empty((n * n, d_v), dtype=np.float64) if want_dvalues else None
        dw = np.empty((T, H, k), dtype=np.float64)
        ds = np.empty((T, H, k), dtype=np.float64)
        rc = self.lib.pkm_oracle_backward(T, H, n, k, d_k, d_v, qp, qd, kp, kd, vp, vd,
                                          self._ptr(idx), self._ptr(weights), dyp, dyd,
                                          self._ptr(dq), self._ptr(dkeys), self._ptr(dvalues),
                                          self._ptr(dw), self._ptr(ds), nthreads)
        if rc != 0:
            raise RuntimeError(f"pkm_oracle_backward failed: {rc}")
        return dict(dq=dq, dkeys=dkeys, dvalues=dvalues, dw=dw, ds=ds)


_default = None


def default() -> Oracle:
    """The oracle built in place (compiled on first use if missing)."""
    global _default
    if _default is None:
        if not os.path.exists(LIB_PATH):
            build()
        _default = Oracle(LIB_PATH)
    return _default
