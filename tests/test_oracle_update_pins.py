"""Pins of the update/usage oracle (oracle/update.py) against hand-computed
values and closed forms: a plausible mistake (a sign, an untouched row
written, a missing bias correction, a wrong rounding) fails one of them."""
import numpy as np

from oracle import update as U


def test_usage_hand_example():
    # n = 2 (slots 0..3); batch 1: picks 0, 3, 3, 1; batch 2: picks 2, 3
    b1 = np.array([[[0, 3]], [[3, 1]]])
    b2 = np.array([[[2, 3]]])
    counts, used = U.slot_usage([b1], 2)
    assert counts.tolist() == [1, 1, 0, 2] and used == 3
    counts, used = U.slot_usage([b1, b2], 2)
    assert counts.tolist() == [1, 1, 1, 3] and used == 4


def test_usage_invariants():
    rng = np.random.default_rng(5)
    batches = [rng.integers(0, 100, size=(7, 3, 4)) for _ in range(3)]
    counts, used = U.slot_usage(batches, 10)
    assert counts.sum() == 3 * 7 * 3 * 4
    assert used == len(np.unique(np.concatenate([b.ravel() for b in batches])))
    assert np.array_equal(U.touched_slots(batches, 10), counts > 0)


def test_sgd_closed_forms_fp32():
    vals = np.array([[1.0, -2.0], [3.0, 4.0], [5.0, 6.0]], dtype=np.float32)
    grads = np.array([[0.5, 1.0], [8.0, 8.0], [2.0, -2.0]], dtype=np.float32)
    touched = np.array([True, False, True])
    out = U.sparse_sgd(vals, grads, touched, 0.5)
    assert out.tolist() == [[0.75, -2.5], [3.0, 4.0], [4.0, 7.0]]
    assert np.array_equal(U.sparse_sgd(vals, grads, touched, 0.0), vals)


def test_sgd_bf16_rounding():
    one = np.array([[0x3F80, 0x3F80]], dtype=np.uint16)          # 1.0, 1.0
    g = np.array([[2.0 ** -9, 3 * 2.0 ** -10]], dtype=np.float32)
    out = U.sparse_sgd(one, g, np.array([True]), 1.0)
    # 1 - 2^-9 sits halfway between 1 - 2^-8 (odd) and 1.0 (even): ties to 1.0;
    # 1 - 3*2^-10 is below the midpoint: 1 - 2^-8 = 0x3F7F
    assert out.tolist() == [[0x3F80, 0x3F7F]]
    assert np.array_equal(U.sparse_sgd(one, g, np.array([False]), 1.0), one)


def test_adam_first_step_closed_form():
    # from zero moments, step 1: m/c1 = g, v/c2 = g^2, so the step is g / (|g| + eps)
    rng = np.random.default_rng(6)
    w = rng.standard_normal((4, 8)).astype(np.float32)
    g = rng.standard_normal((4, 8)).astype(np.float32)
    z = np.zeros_like(w)
    touched = np.array([True, True, False, True])
    lr, eps = 0.01, 1e-8
    out, m, v = U.sparse_adam(w, g, touched, z, z, 1, lr, 0.9, 0.999, eps)
    want = w.astype(np.float64) - lr * g / (np.abs(g) + eps)
    assert np.allclose(out[touched], want[touched], rtol=0, atol=1e-6)
    assert np.array_equal(out[~touched], w[~touched])
    # the moments' weights are those of the float32 constants the boundary takes
    b1, b2 = float(np.float32(0.9)), float(np.float32(0.999))
    assert np.allclose(m[touched], (1 - b1) * g[touched].astype(np.float64), rtol=1e-6)
    assert np.allclose(v[touched], (1 - b2) * g[touched].astype(np.float64) ** 2, rtol=1e-6)
    assert np.array_equal(m[~touched], z[~touched]) and np.array_equal(v[~touched], z[~touched])


def test_adam_lazy_rows_keep_their_moments():
    # a row not selected at step 2 keeps step 1's moments and value
    w = np.ones((2, 8), dtype=np.float32)
    g = np.full((2, 8), 0.5, dtype=np.float32)
    z = np.zeros_like(w)
    w1, m1, v1 = U.sparse_adam(w, g, np.array([True, True]), z, z, 1, 0.1, 0.9, 0.999, 1e-8)
    w2, m2, v2 = U.sparse_adam(w1, g, np.array([True, False]), m1, v1, 2, 0.1, 0.9, 0.999, 1e-8)
    assert np.array_equal(w2[1], w1[1]) and np.array_equal(m2[1], m1[1])
    assert np.array_equal(v2[1], v1[1])
    # the selected row: m = 0.9 * 0.05 + 0.1 * 0.5 = 0.095; c1 = 1 - 0.81 = 0.19 -> m/c1 = 0.5
    assert np.allclose(m2[0], 0.095, rtol=1e-6)
    assert np.allclose(w2[0], w1[0] - 0.1 * 0.5 / (0.5 + 1e-8), atol=1e-6)
