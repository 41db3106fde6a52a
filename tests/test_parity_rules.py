"""The comparison rules of the GPU parity tests, checked on the CPU: a float32
emulation of the gather passes the element-wise y bound, a planted error of one
bfloat16 spacing or a wrong element fails it; a float32 evaluation of the
gradients passes the gradient checks with their summation allowance, a
dropped or sign-flipped pick fails them (no GPU)."""
import numpy as np
import pytest

import gpu_util
import parity
import pkm_inputs


def _emulate(dtype, seed=3, T=40, H=3, n=12, k=5, d_v=24):
    rng = np.random.default_rng(seed)
    inp = pkm_inputs.custom(T, H, n, k, 16, d_v, dtype=dtype, seed=seed)
    vals = gpu_util.bits_to_f64(inp["values"])
    idx = np.stack([np.stack([rng.choice(n * n, k, replace=False) for _ in range(H)])
                    for _ in range(T)]).astype(np.int32)
    w_ref = rng.random((T, H, k))
    w_ref /= w_ref.sum(axis=2, keepdims=True)
    w_gpu = w_ref.astype(np.float32)                      # what a float32 softmax stores
    exact = np.einsum("thr,thrc->tc", w_ref, vals[idx])
    acc = np.zeros((T, d_v), np.float32)
    for h in range(H):                                    # float32 multiply-adds, pick order
        for r in range(k):
            acc = (acc + w_gpu[:, h, r:r + 1] * vals[idx[:, h, r]].astype(np.float32)).astype(np.float32)
    if dtype == "bf16":
        got = gpu_util.bits_to_f64(pkm_inputs.bf16_bits(acc))
    else:
        got = acc.astype(np.float64)
    bound = gpu_util.y_sum_bound(inp["values"], idx, w_gpu, w_ref)
    return got, exact, bound


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_y_bound_accepts_float32_sums(dtype):
    got, exact, bound = _emulate(dtype)
    assert parity.assert_y_bound("y", got, exact, bound, dtype) <= 1.0
    assert parity.assert_elems_close("y", got, exact, parity.TOL[dtype]) <= parity.TOL[dtype]


def test_y_bound_rejects_one_bf16_spacing():
    got, exact, bound = _emulate("bf16")
    bad = got.copy()
    bad[7, 3] += parity.bf16_ulp(np.array(exact[7, 3]))   # one whole spacing too far
    with pytest.raises(AssertionError):
        parity.assert_y_bound("y", bad, exact, bound, "bf16")


def test_elementwise_rule_catches_one_wrong_element():
    rng = np.random.default_rng(5)
    want = rng.standard_normal((50, 256))
    got = want * (1 + 1e-6)
    assert parity.assert_elems_close("g", got, want, 1e-4) <= 1e-4
    got[10, 17] += 0.05 * np.sqrt(np.mean(want[10] ** 2)) + 0.0 * want[10, 17]
    # row L2 passes (one element of 256 off by 5% of the rms: 0.3% of the row)
    assert parity.row_rel_err(got, want).max() < 2e-2
    with pytest.raises(AssertionError):
        parity.assert_elems_close("g", got, want, 2e-2)


def test_bf16_ulp():
    assert parity.bf16_ulp(np.array(1.0)) == 2.0 ** -7
    assert parity.bf16_ulp(np.array(1.5)) == 2.0 ** -7
    assert parity.bf16_ulp(np.array(0.75)) == 2.0 ** -8
    assert parity.bf16_ulp(np.array(-3.0)) == 2.0 ** -6


# the seeded two-kernel edge case whose sub-key gradients cancel: tokens whose
# k picks share a right sub-key add sum_e ds_e ~ 0 to that sub-key's row
GRAD_CASE = (50, 2, 128, 16, 512, 16)


def _grad_case(orc):
    T, H, n, k, d_k, d_v = GRAD_CASE
    inp = pkm_inputs.custom(T, H, n, k, d_k, d_v, dtype="fp32", seed=T * 131 + n + 7)
    ref = orc.forward(inp["q"], inp["keys"], inp["values"], k)
    idx = ref["idx"]
    w = ref["weights"].astype(np.float32).astype(np.float64)     # float32 weights
    ob = orc.backward(inp["q"], inp["keys"], inp["values"], idx, w, inp["dy"])
    allow = parity.grad_sum_bound(inp["q"], inp["keys"], inp["values"], idx, w, inp["dy"])
    return inp, idx, w, ob, allow


def _f32_grads(inp, idx, w):
    """dq and dkeys evaluated in float32: dw, s, ds, then the sums in pick order."""
    T, H, k = idx.shape
    n, half = inp["keys"].shape[2], inp["keys"].shape[3]
    q = inp["q"].astype(np.float32).reshape(T, H, 2, half)
    keys, vals, dy = (inp[x].astype(np.float32) for x in ("keys", "values", "dy"))
    w32 = w.astype(np.float32)
    dw = np.einsum("thec,tc->the", vals[idx], dy).astype(np.float32)
    s = np.sum(w32 * dw, axis=2, keepdims=True, dtype=np.float32)
    ds = (w32 * (dw - s)).astype(np.float32)
    dq = np.zeros((T, H, 2, half), np.float32)
    dk = np.zeros((H, 2, n, half), np.float32)
    for h in range(H):
        for side, sub in ((0, idx[:, h] // n), (1, idx[:, h] % n)):
            for e in range(k):
                dq[:, h, side] = (dq[:, h, side] + ds[:, h, e:e + 1] * keys[h, side, sub[:, e]]).astype(np.float32)
            contrib = (ds[:, h, :, None] * q[:, h, None, side]).astype(np.float32)
            np.add.at(dk[h, side], sub.reshape(-1), contrib.reshape(-1, half))
    return dq.reshape(T, H, -1).astype(np.float64), dk.astype(np.float64), ds


def test_grad_bound_accepts_float32_gradients(orc):
    inp, idx, w, ob, allow = _grad_case(orc)
    dq, dk, _ = _f32_grads(inp, idx, w)
    half = dk.shape[-1]
    # the bound itself holds element by element
    assert np.all(np.abs(dk - ob["dkeys"]) <= allow["dkeys"])
    assert np.all(np.abs(dq - ob["dq"]) <= allow["dq"])
    tol = parity.TOL["fp32"]
    a_dk = allow["dkeys"].reshape(-1, half)
    parity.assert_rows_close("dkeys", dk.reshape(-1, half), ob["dkeys"].reshape(-1, half), tol, allow=a_dk)
    parity.assert_elems_close("dkeys", dk.reshape(-1, half), ob["dkeys"].reshape(-1, half), tol, allow=a_dk)
    parity.assert_rows_close("dq", dq, ob["dq"], tol, allow=allow["dq"])
    parity.assert_elems_close("dq", dq, ob["dq"], tol, allow=allow["dq"])


@pytest.mark.parametrize("mistake", ["drop", "flip"])
def test_grad_bound_rejects_one_wrong_pick(orc, mistake):
    inp, idx, w, ob, allow = _grad_case(orc)
    T, H, n, k, d_k, d_v = GRAD_CASE
    half = d_k // 2
    tol = parity.TOL["fp32"]
    ds = ob["ds"]
    t, h, e = np.unravel_index(int(np.argmax(np.abs(ds))), ds.shape)
    i, j = divmod(int(idx[t, h, e]), n)
    f = 1.0 if mistake == "drop" else 2.0                 # remove the term, or reverse it
    q = inp["q"].astype(np.float64).reshape(T, H, 2, half)
    bad_dk = ob["dkeys"].copy()
    bad_dk[h, 0, i] -= f * ds[t, h, e] * q[t, h, 0]
    with pytest.raises(AssertionError):
        parity.assert_rows_close("dkeys", bad_dk.reshape(-1, half), ob["dkeys"].reshape(-1, half), tol,
                                 allow=allow["dkeys"].reshape(-1, half))
    bad_dq = ob["dq"].copy()
    bad_dq[t, h, half:] -= f * ds[t, h, e] * inp["keys"][h, 1, j].astype(np.float64)
    with pytest.raises(AssertionError):
        parity.assert_rows_close("dq", bad_dq, ob["dq"], tol, allow=allow["dq"])
