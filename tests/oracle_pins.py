"""Pins of the CPU oracle to things other than itself.

Every check takes an ``oracle.Oracle`` handle, so the same checks run against
the real oracle (``test_oracle_pins.py``) and against deliberately broken
copies of it (``test_oracle_mutants.py``, which shows that each planted mistake
fails at least one check).

What pins what:
  key_identity      explicit concatenated keys (section "Implied keys vs stored
                    sub-keys" of "Product Keys Give Transformers Million-Slot
                    Memory Layers") scored with numpy -> flat scores
  flat_bruteforce   numpy lexsort over explicit keys -> selection, order, gaps
  product_key       the pages' product-key search (top-k per half, k x k
                    combine; section "Why top-k of each half is enough") must
                    give exactly the flat result, ties included
  toy_golden        a hand-derived 3 x 3 example (tests/golden/toy_3x3.json)
  tie_closed_form   right half of q zero -> every right score ties
  k1_exact          k = 1 -> weight 1 and y = the argmax value row, bit-exact
  all_keys_softmax  k = n^2 -> scipy softmax over all keys, y = w @ values
  softmax_props     weights sum to 1 and follow the score order
  multihead_sum     H heads = sum of the H single-head layers
  bwd_invariants    sum_r ds = 0; column sums of dvalues = H * sum_t dy;
                    unselected rows exactly 0
  finite_diff       central differences of L = sum <dy, y> in float64
  linearity         y linear in values; dvalues independent of values
  given_idx         forward on a given selection: forward()'s own result on
                    its own selection, explicit-key recomputation on others
"""
from __future__ import annotations

import json
import os

import numpy as np
import scipy.special

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ---------------------------------------------------------------------------
# independent numpy references (float64)
# ---------------------------------------------------------------------------
def explicit_keys(keys: np.ndarray, h: int) -> np.ndarray:
    """All n*n implied keys of head h, row f = i*n + j = C[i] ++ C'[j]."""
    c0 = np.asarray(keys[h, 0], dtype=np.float64)
    c1 = np.asarray(keys[h, 1], dtype=np.float64)
    n = c0.shape[0]
    return np.concatenate([np.repeat(c0, n, axis=0), np.tile(c1, (n, 1))], axis=1)


def np_flat(q, keys, k):
    """Flat search over explicit keys: idx, sorted scores per (t, h)."""
    q = np.asarray(q, dtype=np.float64)
    T, H, _ = q.shape
    n = keys.shape[2]
    idx = np.empty((T, H, k), dtype=np.int64)
    sc = np.empty((T, H, n * n))
    for h in range(H):
        S = q[:, h, :] @ explicit_keys(keys, h).T
        for t in range(T):
            order = np.lexsort((np.arange(n * n), -S[t]))
            idx[t, h] = order[:k]
            sc[t, h] = S[t, order]
    return idx, sc


def np_product_key(q, keys, k):
    """Product-key search: exact top-k per half, then the best k of the pairs."""
    q = np.asarray(q, dtype=np.float64)
    T, H, d_k = q.shape
    n = keys.shape[2]
    half = d_k // 2
    kk = min(k, n)
    idx = np.empty((T, H, k), dtype=np.int64)
    for t in range(T):
        for h in range(H):
            s1 = np.asarray(keys[h, 0], np.float64) @ q[t, h, :half]
            s2 = np.asarray(keys[h, 1], np.float64) @ q[t, h, half:]
            L = np.lexsort((np.arange(n), -s1))[:kk]
            R = np.lexsort((np.arange(n), -s2))[:kk]
            cand_f = (L[:, None] * n + R[None, :]).ravel()
            cand_s = (s1[L][:, None] + s2[R][None, :]).ravel()
            idx[t, h] = cand_f[np.lexsort((cand_f, -cand_s))[:k]]
    return idx


def rand_problem(rng, T, H, n, d_k, d_v, integer=False, dup_rows=False):
    if integer:
        q = rng.integers(-3, 4, size=(T, H, d_k)).astype(np.float64)
        keys = rng.integers(-2, 3, size=(H, 2, n, d_k // 2)).astype(np.float64)
    else:
        q = rng.standard_normal((T, H, d_k))
        keys = rng.standard_normal((H, 2, n, d_k // 2))
    if dup_rows and n >= 3:
        keys[:, 0, n - 1] = keys[:, 0, 0]
        keys[:, 1, 1] = keys[:, 1, n - 2]
    values = rng.standard_normal((n * n, d_v))
    return q, keys, values


# ---------------------------------------------------------------------------
# the pins
# ---------------------------------------------------------------------------
def pin_key_identity(o):
    rng = np.random.default_rng(11)
    q, keys, _ = rand_problem(rng, 3, 2, 7, 10, 3)
    for t in range(3):
        for h in range(2):
            got = o.flat_scores(q, keys, t, h)
            want = explicit_keys(keys, h) @ q[t, h]
            assert np.allclose(got, want, rtol=1e-12, atol=1e-12), "flat scores != <q, C_i ++ C'_j>"


def pin_flat_bruteforce(o):
    rng = np.random.default_rng(12)
    for (T, H, n, d_k, k) in [(5, 1, 4, 6, 3), (4, 2, 5, 4, 7), (3, 3, 6, 8, 1), (3, 1, 3, 2, 9)]:
        q, keys, values = rand_problem(rng, T, H, n, d_k, 2)
        r = o.forward(q, keys, values, k)
        idx, sc = np_flat(q, keys, k)
        assert np.array_equal(r["idx"], idx), "selection/order differs from brute force"
        assert np.allclose(r["scores"], sc[:, :, :k], rtol=1e-12, atol=1e-12), "scores differ"
        assert np.allclose(r["kth"], sc[:, :, k - 1], rtol=1e-12, atol=1e-12), "k-th score"
        want1 = sc[:, :, k] if k < n * n else np.full((T, H), -np.inf)
        assert np.allclose(r["kth1"], want1, rtol=1e-12, atol=1e-12), "(k+1)-th score"


def pin_product_key(o):
    rng = np.random.default_rng(13)
    cases = []
    for n in (2, 3, 5, 8, 17):
        for k in sorted({1, 2, n // 2 + 1, n}):
            cases.append((n, k))
    for case_no, (n, k) in enumerate(cases):
        H = 1 + case_no % 3
        for integer, dup in ((False, False), (True, False), (True, True)):
            q, keys, values = rand_problem(rng, 4, H, n, 6, 2, integer=integer, dup_rows=dup)
            r = o.forward(q, keys, values, k)
            want = np_product_key(q, keys, k)
            assert np.array_equal(r["idx"], want), f"product-key search differs (n={n} k={k} int={integer})"
            flat_idx, _ = np_flat(q, keys, k)
            assert np.array_equal(r["idx"], flat_idx)


def load_toy():
    with open(os.path.join(GOLDEN, "toy_3x3.json")) as f:
        g = json.load(f)
    q = np.array(g["q"], dtype=np.float64)
    keys = np.array(g["keys"], dtype=np.float64)
    values = np.array([[f, 10 - f] for f in range(9)], dtype=np.float64)
    return g, q, keys, values


def pin_toy_golden(o):
    g, q, keys, values = load_toy()
    assert np.array_equal(o.flat_scores(q, keys, 0, 0), np.array(g["flat_scores"], np.float64))
    e = np.e
    for k in (1, 2, 3, 4, 9):
        r = o.forward(q, keys, values, k)
        assert r["idx"][0, 0].tolist() == g["order"][:k], f"toy order k={k}"
    r = o.forward(q, keys, values, 2)
    w0, w1 = e / (1 + e), 1 / (1 + e)
    assert np.allclose(r["weights"][0, 0], [w0, w1], rtol=1e-14)
    assert np.allclose(r["y"][0], [6 * w0 + 3 * w1, 4 * w0 + 7 * w1], rtol=1e-14)
    r3 = o.forward(q, keys, values, 3)
    z = 1 + e ** -1 + e ** -2
    assert np.allclose(r3["weights"][0, 0], [1 / z, e ** -1 / z, e ** -2 / z], rtol=1e-14)
    b = o.backward(q, keys, values, r["idx"], r["weights"], np.array([[1.0, 0.0]]))
    c = 3 * w0 * w1
    assert np.allclose(b["dw"][0, 0], [6, 3], rtol=1e-14)
    assert np.allclose(b["ds"][0, 0], [c, -c], rtol=1e-12)
    assert np.allclose(b["dq"][0, 0], [c, 0, 0, 0], rtol=1e-12, atol=1e-14)
    dk = np.zeros((1, 2, 3, 2))
    dk[0, 0, 2] = [c, 2 * c]
    dk[0, 0, 1] = [-c, -2 * c]
    assert np.allclose(b["dkeys"], dk, rtol=1e-12, atol=1e-14)
    dv = np.zeros((9, 2))
    dv[6] = [w0, 0]
    dv[3] = [w1, 0]
    assert np.allclose(b["dvalues"], dv, rtol=1e-14, atol=0)


def pin_tie_closed_form(o):
    rng = np.random.default_rng(14)
    n, k, d_k = 9, 4, 8
    q, keys, values = rand_problem(rng, 5, 1, n, d_k, 3)
    q[:, :, d_k // 2:] = 0.0
    r = o.forward(q, keys, values, k)
    for t in range(5):
        s1 = keys[0, 0] @ q[t, 0, :d_k // 2]
        i_star = int(np.lexsort((np.arange(n), -s1))[0])
        assert r["idx"][t, 0].tolist() == [i_star * n + j for j in range(k)], "tie-break on right ties"
        assert np.allclose(r["weights"][t, 0], 1.0 / k, rtol=1e-15)
        assert np.allclose(r["y"][t], values[i_star * n: i_star * n + k].mean(axis=0), rtol=1e-13)


def pin_k1_exact(o):
    rng = np.random.default_rng(15)
    q, keys, values = rand_problem(rng, 6, 1, 8, 6, 5)
    q32, k32, v32 = q.astype(np.float32), keys.astype(np.float32), values.astype(np.float32)
    r = o.forward(q32, k32, v32, 1)
    idx, _ = np_flat(q32.astype(np.float64), k32.astype(np.float64), 1)
    assert np.array_equal(r["idx"], idx)
    assert np.all(r["weights"] == 1.0)
    assert np.array_equal(r["y"], v32[idx[:, 0, 0]].astype(np.float64)), "k=1 output must be the row itself"


def pin_all_keys_softmax(o):
    rng = np.random.default_rng(16)
    n = 4
    q, keys, values = rand_problem(rng, 3, 1, n, 4, 3)
    r = o.forward(q, keys, values, n * n)
    for t in range(3):
        s = explicit_keys(keys, 0) @ q[t, 0]
        w = scipy.special.softmax(s)
        assert np.allclose(r["y"][t], w @ values, rtol=1e-12, atol=1e-14)
        assert np.allclose(np.sort(r["weights"][t, 0]), np.sort(w), rtol=1e-12)


def pin_softmax_props(o):
    rng = np.random.default_rng(17)
    q, keys, values = rand_problem(rng, 8, 2, 6, 6, 2)
    r = o.forward(q, keys, values, 5)
    assert np.allclose(r["weights"].sum(axis=2), 1.0, rtol=0, atol=1e-14)
    assert np.all(np.diff(r["weights"], axis=2) <= 1e-16), "weights must follow the score order"
    assert np.all(np.diff(r["scores"], axis=2) <= 0)
    # exp(score difference) = weight ratio
    ratio = r["weights"][:, :, 1:] / r["weights"][:, :, :1]
    assert np.allclose(ratio, np.exp(r["scores"][:, :, 1:] - r["scores"][:, :, :1]), rtol=1e-12)


def pin_multihead_sum(o):
    rng = np.random.default_rng(18)
    H = 3
    q, keys, values = rand_problem(rng, 4, H, 5, 6, 4)
    r = o.forward(q, keys, values, 3)
    total = np.zeros_like(r["y"])
    for h in range(H):
        rh = o.forward(q[:, h:h + 1].copy(), keys[h:h + 1].copy(), values, 3)
        assert np.array_equal(rh["idx"][:, 0], r["idx"][:, h])
        total += rh["y"]
    assert np.allclose(r["y"], total, rtol=1e-13, atol=1e-14)


def pin_bwd_invariants(o):
    rng = np.random.default_rng(19)
    T, H, n, d_v = 9, 2, 6, 4
    q, keys, values = rand_problem(rng, T, H, n, 6, d_v)
    dy = rng.standard_normal((T, d_v))
    r = o.forward(q, keys, values, 4)
    b = o.backward(q, keys, values, r["idx"], r["weights"], dy)
    assert np.allclose(b["ds"].sum(axis=2), 0.0, atol=1e-13), "softmax backward must sum to 0"
    assert np.allclose(b["dvalues"].sum(axis=0), H * dy.sum(axis=0), rtol=1e-12, atol=1e-13)
    touched = np.zeros(n * n, bool)
    touched[r["idx"].ravel()] = True
    assert np.all(b["dvalues"][~touched] == 0.0), "unselected value rows must get exact zeros"
    for t in range(T):
        for h in range(H):
            for rr in range(4):
                assert np.isclose(b["dw"][t, h, rr], dy[t] @ values[r["idx"][t, h, rr]], rtol=1e-12)


def _loss(o, q, keys, values, dy, k):
    r = o.forward(q, keys, values, k)
    return float((r["y"] * dy).sum()), r["idx"]


def pin_finite_diff(o):
    rng = np.random.default_rng(20)
    T, H, n, d_k, d_v, k = 6, 2, 5, 6, 3, 3
    q, keys, values = rand_problem(rng, T, H, n, d_k, d_v)
    dy = rng.standard_normal((T, d_v))
    r = o.forward(q, keys, values, k)
    b = o.backward(q, keys, values, r["idx"], r["weights"], dy)
    eps = 1e-6
    for name, grad in (("q", b["dq"]), ("keys", b["dkeys"]), ("values", b["dvalues"])):
        for trial in range(3):
            args = {"q": q, "keys": keys, "values": values}
            v = rng.standard_normal(args[name].shape)
            plus = dict(args)
            minus = dict(args)
            plus[name] = args[name] + eps * v
            minus[name] = args[name] - eps * v
            lp, ip = _loss(o, plus["q"], plus["keys"], plus["values"], dy, k)
            lm, im = _loss(o, minus["q"], minus["keys"], minus["values"], dy, k)
            assert np.array_equal(ip, r["idx"]) and np.array_equal(im, r["idx"]), "selection moved"
            fd = (lp - lm) / (2 * eps)
            an = float((grad * v).sum())
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), f"d/d{name}: fd {fd} vs analytic {an}"


def pin_linearity(o):
    rng = np.random.default_rng(21)
    q, keys, v1 = rand_problem(rng, 5, 2, 4, 4, 3)
    v2 = rng.standard_normal(v1.shape)
    dy = rng.standard_normal((5, 3))
    r1 = o.forward(q, keys, v1, 3)
    r2 = o.forward(q, keys, v2, 3)
    r12 = o.forward(q, keys, 2.0 * v1 - 0.5 * v2, 3)
    assert np.allclose(r12["y"], 2.0 * r1["y"] - 0.5 * r2["y"], rtol=1e-12, atol=1e-13)
    b1 = o.backward(q, keys, v1, r1["idx"], r1["weights"], dy)
    b2 = o.backward(q, keys, v2, r1["idx"], r1["weights"], dy)
    assert np.array_equal(b1["dvalues"], b2["dvalues"]), "dvalues must not depend on values"


def pin_given_idx(o):
    """forward_given_idx: on forward()'s own selection it must reproduce
    forward()'s scores, weights and y; on any other selection (reversed order,
    random non-top-k slots, repeated across heads) it must equal the plain
    recomputation from explicit keys (section "Implied keys vs stored
    sub-keys"): scores = C_i ++ C'_j against q, a scipy softmax over the given
    k, y = sum over heads of w @ values[idx]."""
    rng = np.random.default_rng(22)
    for (T, H, n, d_k, d_v, k) in [(5, 2, 6, 8, 3, 4), (4, 3, 7, 6, 2, 5), (3, 1, 4, 4, 5, 16)]:
        q, keys, values = rand_problem(rng, T, H, n, d_k, d_v)
        r = o.forward(q, keys, values, k)
        g = o.forward_given_idx(q, keys, values, r["idx"])
        assert np.allclose(g["scores"], r["scores"], rtol=1e-14, atol=1e-14), "given own idx: scores"
        assert np.allclose(g["weights"], r["weights"], rtol=1e-14, atol=1e-15), "given own idx: weights"
        assert np.allclose(g["y"], r["y"], rtol=1e-13, atol=1e-14), "given own idx: y"
        for kind in ("reversed", "random"):
            if kind == "reversed":
                sel = r["idx"][:, :, ::-1].copy()
            else:
                sel = np.stack([np.stack([rng.choice(n * n, size=k, replace=False)
                                          for _ in range(H)]) for _ in range(T)]).astype(np.int32)
            got = o.forward_given_idx(q, keys, values, sel)
            y = np.zeros((T, d_v))
            for t in range(T):
                for h in range(H):
                    s = explicit_keys(keys, h)[sel[t, h]] @ q[t, h]
                    w = scipy.special.softmax(s)
                    assert np.allclose(got["scores"][t, h], s, rtol=1e-12, atol=1e-12), f"{kind}: scores"
                    assert np.allclose(got["weights"][t, h], w, rtol=1e-12, atol=1e-15), f"{kind}: weights"
                    y[t] += w @ values[sel[t, h]]
            assert np.allclose(got["y"], y, rtol=1e-12, atol=1e-13), f"{kind}: y"


ALL_PINS = {name[4:]: fn for name, fn in sorted(globals().items()) if name.startswith("pin_")}


def failing_pins(o) -> list:
    """Names of the pins the given oracle handle fails (empty = all pass)."""
    bad = []
    for name, fn in ALL_PINS.items():
        try:
            fn(o)
        except (AssertionError, RuntimeError, ValueError, IndexError):
            bad.append(name)
    return bad
