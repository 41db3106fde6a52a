"""Shared codebooks (PKM_KEYS_SHARED): one pair keys [2][n][d_k/2] serves every
head, and dkeys [2][n][d_k/2] is the sub-key gradient summed over the heads.
Against the oracle given that pair replicated into every head: the same rules
as every parity test (selection sets, weights, y, dq, dvalues), dkeys against
the oracle's per-head dkeys summed over the heads.  Also against the GPU's own
run on the replicated codebooks: the forward and dq, dvalues bit for bit (the
same arithmetic on the same numbers)."""
import numpy as np
import pytest
import torch

import gpu_util
import parity
import pkm_inputs

pytestmark = pytest.mark.gpu

CASES = [
    # dtype, T, H, n, k, d_k, d_v
    ("fp32", 40, 3, 37, 5, 48, 24),        # the one-kernel selection, fp32 storage
    ("fp32", 100, 3, 200, 20, 512, 24),    # the two-kernel selection, fp32 storage
    ("bf16", 40, 3, 37, 5, 48, 24),
    ("bf16", 100, 3, 300, 20, 512, 24),    # the two-kernel selection
    ("bf16", 2048, 4, 512, 32, 512, 64),   # the benchmark's memory shape
]


@pytest.mark.parametrize("case", CASES, ids=[f"{c[0]}-T{c[1]}H{c[2]}n{c[3]}k{c[4]}dk{c[5]}" for c in CASES])
def test_shared_codebooks(orc, case):
    import product_key_memory_amd as pk
    dtype, T, H, n, k, d_k, d_v = case
    dev = gpu_util.device()
    print(f"[shared keys] {case}", flush=True)
    inp = pkm_inputs.custom(T, H, n, k, d_k, d_v, dtype=dtype, seed=T + 7 * n)
    shared = np.ascontiguousarray(inp["keys"][0])                  # [2][n][d_k/2]
    rep = np.ascontiguousarray(np.broadcast_to(shared, (H,) + shared.shape))
    q, values, dy = (gpu_util.to_dev(inp[x], dev) for x in ("q", "values", "dy"))
    keys_s, keys_r = gpu_util.to_dev(shared, dev), gpu_util.to_dev(rep, dev)
    y, idx, wts, sc = pk.pkm_forward(q, keys_s, values, k)
    dq, dkeys, dvalues = pk.pkm_backward(q, keys_s, values, idx, wts, dy)
    y_r, idx_r, wts_r, _ = pk.pkm_forward(q, keys_r, values, k)
    dq_r, dkeys_r, dvalues_r = pk.pkm_backward(q, keys_r, values, idx_r, wts_r, dy)
    torch.cuda.synchronize()
    assert dkeys.shape == (2, n, d_k // 2)
    for name, a, b in (("idx", idx, idx_r), ("weights", wts, wts_r), ("y", y, y_r), ("dq", dq, dq_r),
                       ("dvalues", dvalues, dvalues_r)):
        assert torch.equal(a, b), f"{name}: shared codebooks differ from the replicated ones"

    g_idx, g_w = gpu_util.to_host(idx), gpu_util.to_host(wts)
    ref = orc.forward(inp["q"], rep, inp["values"], k)
    given = orc.forward_given_idx(inp["q"], rep, inp["values"], g_idx)
    parity.check_selection(g_idx, ref, given, n)
    assert float(np.abs(g_w - given["weights"]).max()) <= 1e-4
    tol = parity.TOL[dtype]
    g_y = gpu_util.bits_to_f64(gpu_util.to_host(y))
    parity.assert_rows_close("y", g_y, given["y"], tol)
    parity.assert_elems_close("y", g_y, given["y"], tol)
    w_in = g_w.astype(np.float64)            # the weights the backward was handed
    ob = orc.backward(inp["q"], rep, inp["values"], g_idx, w_in, inp["dy"])
    allow = parity.grad_sum_bound(inp["q"], shared, inp["values"], g_idx, w_in, inp["dy"], shared=True)
    half = d_k // 2
    parity.assert_rows_close("dq", gpu_util.to_host(dq), ob["dq"], tol, allow=allow["dq"])
    parity.assert_elems_close("dq", gpu_util.to_host(dq), ob["dq"], tol, allow=allow["dq"])
    want = ob["dkeys"].sum(axis=0).reshape(-1, half)
    got = gpu_util.to_host(dkeys).reshape(-1, half)
    a_dk = allow["dkeys"].reshape(-1, half)
    parity.assert_rows_close("dkeys (summed over heads)", got, want, tol, allow=a_dk)
    parity.assert_elems_close("dkeys (summed over heads)", got, want, tol, allow=a_dk)
    # the fold over heads against the per-head sub-key gradient of the replicated run
    summed = dkeys_r.double().sum(dim=0).cpu().numpy().reshape(-1, half)
    parity.assert_rows_close("dkeys vs replicated", got, summed, 1e-5)
    touched = np.zeros(n * n, bool)
    touched[g_idx.ravel()] = True
    g_dv = gpu_util.to_host(dvalues)
    assert np.all(g_dv[~touched] == 0)
    parity.assert_rows_close("dvalues", g_dv[touched], ob["dvalues"][touched], tol)
