"""Helpers for the GPU tests: numpy <-> torch and one parity run."""
from __future__ import annotations

import numpy as np
import torch

import parity


def device():
    assert torch.cuda.is_available(), "GPU tests need a GPU (run them with -m gpu on an MI355X)"
    return torch.device("cuda", 0)


def to_dev(a: np.ndarray, dev) -> torch.Tensor:
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def to_host(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def bits_to_f64(a: np.ndarray) -> np.ndarray:
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def y_sum_bound(values: np.ndarray, idx: np.ndarray, w_gpu: np.ndarray, w_ref: np.ndarray,
                chunk: int = 64) -> np.ndarray:
    """Per element of y [T][d_v]: how far float32 sums of the GPU's weights
    times the value rows may lie from the exact sum with the exact weights,
        sum over picks of (|w_gpu - w_ref| + gamma |w_gpu|) * |values[f][c]|,
    gamma = (H k + 2) 2^-24 (with 1% slack): the classic bound on n rounded
    multiply-adds, any order."""
    T, H, k = idx.shape
    d_v = values.shape[1]
    wg = w_gpu.astype(np.float64)
    gamma = 1.01 * (H * k + 2) * 2.0 ** -24
    a = (np.abs(wg - w_ref) + gamma * np.abs(wg)).reshape(T, H * k)
    out = np.empty((T, d_v))
    for t0 in range(0, T, chunk):
        t1 = min(T, t0 + chunk)
        rows = np.abs(bits_to_f64(values[idx[t0:t1].reshape(-1)])).reshape(t1 - t0, H * k, d_v)
        out[t0:t1] = np.einsum("tp,tpc->tc", a[t0:t1], rows)
    return out


def run_parity(orc, inp: dict, k: int, subset=None, backward: bool = False, tol=None,
               tight=None, nthreads: int = 0) -> dict:
    """Run the GPU path on all of inp's tokens; check `subset` (all if None)
    against the oracle.  Returns a report dict."""
    import product_key_memory_amd as pk

    dev = device()
    w = inp["w"]
    n = w.n
    tol = parity.TOL[w.dtype] if tol is None else tol
    q, keys, values = (to_dev(inp[x], dev) for x in ("q", "keys", "values"))
    print(f"[parity] {w.name} T={w.T} H={w.H} n={n} k={k} d_k={w.d_k} d_v={w.d_v} {w.dtype}",
          flush=True)
    y, idx, wts, sc = pk.pkm_forward(q, keys, values, k)
    torch.cuda.synchronize()
    sub = np.arange(w.T) if subset is None else np.asarray(subset)
    g_idx = to_host(idx)[sub]
    g_w = to_host(wts)[sub]
    g_sc = to_host(sc)[sub]
    g_y = bits_to_f64(to_host(y))[sub]
    q_sub = inp["q"][sub]
    ref = orc.forward(q_sub, inp["keys"], inp["values"], k, nthreads=nthreads)
    given = orc.forward_given_idx(q_sub, inp["keys"], inp["values"], g_idx, nthreads=nthreads)
    rep = parity.check_selection(g_idx, ref, given, n)
    werr = float(np.abs(g_w - given["weights"]).max())
    assert werr <= 1e-4, f"weights differ by {werr:.3e}"
    serr = float((np.abs(g_sc - given["scores"]) / np.maximum(1.0, np.abs(given["scores"]))).max())
    assert serr <= 1e-4, f"scores differ by {serr:.3e}"
    rep["w_err"], rep["score_err"] = werr, serr
    rep["y_err"] = parity.assert_rows_close("y", g_y, given["y"], tol)
    rep["y_elem_err"] = parity.assert_elems_close("y", g_y, given["y"], tol)
    bound = y_sum_bound(inp["values"], g_idx, g_w, given["weights"])
    rep["y_bound_ratio"] = parity.assert_y_bound("y", g_y, given["y"], bound, w.dtype)
    if tight is not None:
        assert rep["y_err"] <= tight["y"], f"y error {rep['y_err']:.3e} above the expected {tight['y']}"
    if backward:
        dy_np = inp["dy"]
        mask = np.zeros(w.T, bool)
        mask[sub] = True
        dy_masked = dy_np.copy()
        dy_masked[~mask] = 0
        dq, dkeys, dvalues = pk.pkm_backward(q, keys, values, idx, wts, to_dev(dy_masked, dev))
        torch.cuda.synchronize()
        # the backward is a function of the weights it is handed: the oracle
        # evaluates it at the same (float32) weights as the GPU
        w_in = g_w.astype(np.float64)
        ob = orc.backward(q_sub, inp["keys"], inp["values"], g_idx, w_in, dy_np[sub],
                          nthreads=nthreads)
        allow = parity.grad_sum_bound(q_sub, inp["keys"], inp["values"], g_idx, w_in, dy_np[sub])
        # size of one term of each gradient's sums (see parity.row_rel_err)
        half = w.d_k // 2
        wdw = np.sqrt(np.mean((given["weights"] * ob["dw"]) ** 2))
        rms_row = lambda a: float(np.sqrt(np.mean(np.sum(a * a, axis=1))))  # noqa: E731
        term = {"dq": wdw * rms_row(bits_to_f64(inp["keys"]).reshape(-1, half)),
                "dkeys": wdw * rms_row(bits_to_f64(q_sub).reshape(-1, half)),
                "dvalues": float(np.sqrt(np.mean(given["weights"] ** 2)))
                * rms_row(bits_to_f64(dy_np[sub]))}
        g_dq = to_host(dq)[sub]
        rep["dq_err"] = parity.assert_rows_close("dq", g_dq, ob["dq"], tol,
                                                 abs_floor=1e-3 * term["dq"], allow=allow["dq"])
        rep["dq_elem_err"] = parity.assert_elems_close("dq", g_dq, ob["dq"], tol,
                                                       abs_floor=1e-3 * term["dq"], allow=allow["dq"])
        g_dk = to_host(dkeys).reshape(-1, half)
        a_dk = allow["dkeys"].reshape(-1, half)
        rep["dkeys_err"] = parity.assert_rows_close("dkeys", g_dk, ob["dkeys"].reshape(-1, half), tol,
                                                    abs_floor=1e-3 * term["dkeys"], allow=a_dk)
        rep["dkeys_elem_err"] = parity.assert_elems_close("dkeys", g_dk,
                                                          ob["dkeys"].reshape(-1, half), tol,
                                                          abs_floor=1e-3 * term["dkeys"], allow=a_dk)
        g_dv = to_host(dvalues)
        touched = np.zeros(n * n, bool)
        touched[g_idx.ravel()] = True
        assert np.all(g_dv[~touched] == 0.0), "unselected value rows must stay exactly 0"
        rows = np.nonzero(touched)[0]
        rep["dvalues_err"] = parity.assert_rows_close("dvalues", g_dv[rows], ob["dvalues"][rows], tol,
                                                      abs_floor=1e-3 * term["dvalues"])
        rep["dvalues_elem_err"] = parity.assert_elems_close("dvalues", g_dv[rows],
                                                            ob["dvalues"][rows], tol,
                                                            abs_floor=1e-3 * term["dvalues"])
        if tight is not None:
            # against the typical row size: rows whose own sum nearly cancels
            # (a hot sub-key shared by most picks of a head) amplify float32
            # rounding in the relative measure above, not in this one
            for key, got, want in (("dq", g_dq, ob["dq"]),
                                   ("dkeys", g_dk, ob["dkeys"].reshape(-1, half)),
                                   ("dvalues", g_dv[rows], ob["dvalues"][rows])):
                e = float(parity.row_rel_err(got, want, floor=1.0, abs_floor=term[key]).max())
                rep[key + "_err_vs_rms"] = e
                assert e <= tight["grad"], f"{key}: error {e:.3e} of the rms row above {tight['grad']}"
    print(f"[parity] ok {rep}", flush=True)
    return rep
