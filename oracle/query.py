"""fp64 CPU oracle of the query network -- TEST INFRASTRUCTURE ONLY (same
rules as the rest of ``oracle/``).

The plain definitions (gptget.net summary of "Large Memory Layers with Product
Keys": the query network turns x into q, and batch normalization inside it
raises memory utilization), in float64 with numpy:

    z = x W^T
    mean = (1/T) sum_t z,  var = (1/T) sum_t (z - mean)^2,  rstd = 1/sqrt(var + eps)
    zhat = (z - mean) rstd,  q = gamma zhat + beta

and the gradients of L = sum dq * q written out from the chain rule:

    dbeta = sum_t dq,  dgamma = sum_t dq zhat
    dzhat = gamma dq
    dz = rstd (dzhat - mean_t dzhat - zhat mean_t(dzhat zhat))
    dx = dz W,  dW = dz^T x

Inputs may be float32 or uint16 (raw bfloat16 bits), widened exactly.
"""
from __future__ import annotations

import numpy as np


def _widen(a: np.ndarray) -> np.ndarray:
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return np.asarray(a, dtype=np.float64)


def query_forward(x, W, gamma=None, beta=None, eps: float = 1e-5) -> dict:
    x64, W64 = _widen(x), _widen(W)
    z = x64 @ W64.T
    mean = z.mean(axis=0)
    var = ((z - mean) ** 2).mean(axis=0)
    rstd = 1.0 / np.sqrt(var + np.float64(np.float32(eps)))
    zhat = (z - mean) * rstd
    g = np.ones(z.shape[1]) if gamma is None else np.asarray(gamma, dtype=np.float64)
    b = np.zeros(z.shape[1]) if beta is None else np.asarray(beta, dtype=np.float64)
    return {"z": z, "mean": mean, "var": var, "rstd": rstd, "zhat": zhat, "q": g * zhat + b}


def query_backward(x, W, dq, gamma=None, eps: float = 1e-5) -> dict:
    f = query_forward(x, W, gamma, None, eps)
    x64, W64 = _widen(x), _widen(W)
    dq = np.asarray(dq, dtype=np.float64)
    zhat, rstd = f["zhat"], f["rstd"]
    g = np.ones(zhat.shape[1]) if gamma is None else np.asarray(gamma, dtype=np.float64)
    dzhat = dq * g
    dz = rstd * (dzhat - dzhat.mean(axis=0) - zhat * (dzhat * zhat).mean(axis=0))
    return {"dx": dz @ W64, "dW": dz.T @ x64, "dgamma": (dq * zhat).sum(axis=0),
            "dbeta": dq.sum(axis=0), "dz": dz}
