"""The comparison rules of the GPU parity tests, checked on the CPU: a float32
emulation of the gather passes the element-wise y bound, a planted error of one
bfloat16 spacing or a wrong element fails it (no GPU)."""
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
