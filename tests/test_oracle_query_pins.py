"""Pins of the query-network oracle (oracle/query.py): the projection against
an explicit loop, batch-norm's closed-form output statistics, the affine map,
and finite differences of every gradient; a dropped term, a transposed
operand or a wrong sign fails one of them."""
import numpy as np

from oracle import query as Q


def _case(seed, T=7, dm=5, D=4):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((T, dm)), rng.standard_normal((D, dm)),
            rng.standard_normal(D), rng.standard_normal(D), rng.standard_normal((T, D)))


def test_projection_explicit_loop():
    x, W, _, _, _ = _case(1)
    z = Q.query_forward(x, W)["z"]
    for t in range(x.shape[0]):
        for c in range(W.shape[0]):
            assert abs(z[t, c] - sum(x[t, i] * W[c, i] for i in range(x.shape[1]))) < 1e-12


def test_batchnorm_output_statistics():
    # with gamma = 1, beta = 0 every feature has mean 0 and variance var / (var + eps)
    x, W, _, _, _ = _case(2, T=50)
    f = Q.query_forward(x, W, eps=1e-3)
    assert np.allclose(f["q"].mean(axis=0), 0, atol=1e-12)
    eps32 = float(np.float32(1e-3))
    assert np.allclose(f["q"].var(axis=0), f["var"] / (f["var"] + eps32), rtol=1e-12)


def test_affine_map():
    x, W, g, b, _ = _case(3)
    q0 = Q.query_forward(x, W)["q"]
    assert np.allclose(Q.query_forward(x, W, g, b)["q"], g * q0 + b, atol=1e-12)


def test_gradients_finite_differences():
    x, W, g, b, dq = _case(4)
    eps = 1e-3
    grads = Q.query_backward(x, W, dq, g, eps)

    def loss(x_, W_, g_, b_):
        return float((dq * Q.query_forward(x_, W_, g_, b_, eps)["q"]).sum())

    h = 1e-6
    rng = np.random.default_rng(5)
    for name, arr, idx in (("dx", x, 0), ("dW", W, 1), ("dgamma", g, 2), ("dbeta", b, 3)):
        d = rng.standard_normal(arr.shape)
        args_p = [x, W, g, b]
        args_m = [x, W, g, b]
        args_p[idx] = arr + h * d
        args_m[idx] = arr - h * d
        fd = (loss(*args_p) - loss(*args_m)) / (2 * h)
        an = float((grads[name] * d).sum())
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, fd, an)


def test_dz_removes_mean_and_scale_direction():
    # batch norm's input gradient has zero column sums, and (gamma = 1, eps -> 0)
    # is orthogonal to zhat per column
    x, W, _, _, dq = _case(6, T=40)
    r = Q.query_backward(x, W, dq, None, 1e-12)
    zhat = Q.query_forward(x, W, eps=1e-12)["zhat"]
    assert np.allclose(r["dz"].sum(axis=0), 0, atol=1e-9)
    assert np.allclose((r["dz"] * zhat).sum(axis=0), 0, atol=1e-6)
