"""The C ABI library loads, exports what include/pkm.h declares, and rejects
bad arguments on the host before anything reaches a GPU (no compute calls)."""
import ctypes
import os
import re

import pytest

from product_key_memory_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    with open(os.path.join(ROOT, "include", "pkm.h")) as f:
        text = f.read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_]+\s*\*?\s*(pkm_[a-z_]+)\s*\(", text, re.M)))


def test_exports_every_declared_symbol():
    lib = _lib.lib()
    names = declared_functions()
    assert set(names) == set(_lib.EXPORTS), names
    for name in names:
        assert hasattr(lib, name), name


def test_problem_struct_layout():
    assert ctypes.sizeof(_lib.Problem) == 32


def P(**kw):
    base = dict(T=16, H=2, n=64, k=8, d_k=64, d_v=32, dtype=0)
    base.update(kw)
    return _lib.Problem(base["T"], base["H"], base["n"], base["k"], base["d_k"], base["d_v"], base["dtype"])


FAKE = 1 << 20          # an aligned, never-dereferenced address


@pytest.mark.parametrize("kw,code", [
    (dict(k=0), 2), (dict(k=65, n=128), 2), (dict(k=9, n=8), 2), (dict(n=0), 2), (dict(n=1025), 2),
    (dict(d_k=24), 2), (dict(d_k=8), 2), (dict(d_k=1040), 2), (dict(d_v=12), 2), (dict(d_v=0), 2),
    (dict(H=0), 2), (dict(H=65), 2), (dict(T=-1), 2), (dict(dtype=7), 3),
])
def test_forward_rejects_bad_shapes(kw, code):
    rc = _lib.forward(P(**kw), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, 0, None)
    assert rc == code, _lib.STATUS.get(rc)


def test_dtype_flags():
    """dtype carries the storage type and the shared-codebook flag only."""
    shared = _lib.PKM_KEYS_SHARED
    assert _lib.workspace_bytes(P(dtype=1 | shared), True) == _lib.workspace_bytes(P(dtype=1), True)
    assert _lib.workspace_bytes(P(dtype=1 | 0x200), True) == (1 << 64) - 1
    assert _lib.forward(P(dtype=0x200), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, 0, None) == 3
    assert _lib.forward(P(dtype=2 | shared), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, 0, None) == 3


def test_flat_select_checks():
    """The flat search: bf16 storage only, d_k = 512, n >= 32, k <= 32."""
    ok = dict(d_k=512, n=64, k=8, dtype=1)
    args = [FAKE, FAKE, FAKE, FAKE, None, None]
    assert _lib.flat_forward_select(P(**{**ok, "dtype": 0}), *args) == 3
    assert _lib.flat_forward_select(P(**{**ok, "d_k": 256}), *args) == 2
    assert _lib.flat_forward_select(P(**{**ok, "n": 16}), *args) == 2
    assert _lib.flat_forward_select(P(**{**ok, "k": 33}), *args) == 2
    assert _lib.flat_forward_select(P(**ok), None, FAKE, FAKE, FAKE, None, None) == 1
    assert _lib.flat_forward_select(P(**{**ok, "T": 0}), None, FAKE, None, None, None, None) == 0


def test_null_and_alignment():
    assert _lib.forward(P(), None, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, 0, None) == 1
    assert _lib.forward(P(), FAKE + 4, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, 0, None) == 6
    assert _lib.forward_select(P(), FAKE, FAKE, None, FAKE, None, None, 0, None) == 1
    assert _lib.backward_values(P(), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, FAKE + 8, FAKE,
                                1 << 30, None) == 6
    assert _lib.backward_values(P(), *[FAKE] * 7, 0, FAKE, None, 1 << 30, None) == 1
    assert _lib.backward_values(P(), *[FAKE] * 7, 0, FAKE, FAKE, 16, None) == 4
    assert _lib.slot_sort(P(), FAKE, None, FAKE, FAKE, 1 << 30, None) == 1


def test_backward_workspace_checks():
    p = P()
    need = _lib.workspace_bytes(p, True)
    picks = 16 * 2 * 8
    assert need >= picks * 4 + 64 * 64 * 4 * 3 + picks * 4     # dw + slot sort at least
    assert _lib.workspace_bytes(p, False) == 0       # this shape takes the one-kernel selection
    # the stages that take a workspace reject a 16-byte one
    assert _lib.slot_sort(p, FAKE, FAKE, FAKE, FAKE, 16, None) == 4
    assert _lib.backward_queries(p, *[FAKE] * 7, FAKE, 16, None) == 4
    args = [FAKE] * 9
    for call in (_lib.backward, _lib.backward_overwrite):
        assert call(p, *args, FAKE, need - 1, None) == 4
        assert call(p, *args, None, 0, None) == 1
        assert call(P(d_v=4104), *args, FAKE, 1 << 30, None) == 2   # backward row limit
        assert call(p, *args[:8], None, FAKE, need, None) == 1        # dvalues is required


def test_backward_prototype_is_the_contract():
    """pkm_backward has the contract's 13 parameters -- (p, q, keys, values, idx,
    weights, dy, dq, dkeys, dvalues, workspace, workspace_bytes, stream) with
    dvalues accumulated -- and the overwrite mode is an entry point of its own
    with the same parameters."""
    with open(os.path.join(ROOT, "include", "pkm.h")) as f:
        text = f.read()

    def params(name):
        m = re.search(r"pkm_status_t\s+" + name + r"\s*\(([^)]*)\)", text)
        assert m, name
        return [re.split(r"[\s*]+", a.strip())[-1] for a in m.group(1).split(",")]

    want = ["p", "q", "keys", "values", "idx", "weights", "dy", "dq", "dkeys", "dvalues",
            "workspace", "workspace_bytes", "stream"]
    assert params("pkm_backward") == want
    assert params("pkm_backward_overwrite") == want
    assert "ACCUMULATED" in text.split("pkm_status_t pkm_backward(")[0].rsplit("/*", 1)[1]
    assert len(_lib.lib().pkm_backward.argtypes) == 13


def test_backward_sgd_checks():
    """The fused backward + SGD: its own workspace size (backward = 2), host-side
    argument checks before any launch."""
    p = P()
    need = _lib.workspace_bytes(p, 2)
    assert need >= _lib.workspace_bytes(p, 1)
    assert _lib.workspace_bytes(p, 3) == (1 << 64) - 1
    args = [FAKE] * 8                 # q, keys, values, idx, weights, dy, dq, dkeys
    assert _lib.backward_sgd(p, *args, 0.1, FAKE, need - 1, None) == 4
    assert _lib.backward_sgd(p, *args, float("inf"), FAKE, need, None) == 7
    assert _lib.backward_sgd(p, None, *args[1:], 0.1, FAKE, need, None) == 1
    assert _lib.backward_sgd(p, FAKE, FAKE, FAKE + 8, *args[3:], 0.1, FAKE, need, None) == 6
    assert _lib.backward_sgd(P(d_v=4104), *args, 0.1, FAKE, 1 << 30, None) == 2


def test_workspace_of_invalid_problem():
    assert _lib.workspace_bytes(P(k=0), True) == (1 << 64) - 1


def test_status_strings():
    for code, name in _lib.STATUS.items():
        assert _lib.status_string(code).startswith(name)


def test_forward_workspace_checks():
    """The two-kernel selection (d_k = 512, k <= 32, 128 <= n <= 1024 for bf16
    and 128 <= n <= 256 for float32) keeps its per-half top-k lists in the
    caller's workspace."""
    p = P(T=100, H=3, n=300, k=20, d_k=512, d_v=64, dtype=_lib.PKM_BF16)
    need = _lib.workspace_bytes(p, False)
    assert need == (100 * 3 * 2 * 20 * 8 + 255) // 256 * 256
    args = [FAKE] * 5
    assert _lib.forward_select(p, *args, None, 0, None) == 1
    assert _lib.forward_select(p, *args, FAKE, need - 1, None) == 4
    assert _lib.forward_select(p, *args, FAKE + 8, need, None) == 6
    assert _lib.forward(p, *[FAKE] * 7, FAKE, need - 1, None) == 4
    # other shapes need none, and accept a NULL workspace
    big = P(T=100, H=3, n=1024, k=32, d_k=512, d_v=64, dtype=_lib.PKM_BF16)
    assert _lib.workspace_bytes(big, False) == (100 * 3 * 2 * 32 * 8 + 255) // 256 * 256
    q = P(T=100, H=3, n=300, k=20, d_k=256, d_v=64, dtype=_lib.PKM_BF16)
    assert _lib.workspace_bytes(q, False) == 0
    for n, k in ((127, 20), (1024, 33)):
        assert _lib.workspace_bytes(P(T=100, H=3, n=n, k=k, d_k=512, d_v=64,
                                      dtype=_lib.PKM_BF16), False) == 0
    # float32 storage: the two-kernel path for 128 <= n <= 256 only
    for n, k, on in ((128, 16, True), (256, 32, True), (127, 16, False), (257, 16, False),
                     (200, 33, False)):
        got = _lib.workspace_bytes(P(T=100, H=3, n=n, k=k, d_k=512, d_v=64, dtype=_lib.PKM_FP32),
                                   False)
        assert got == ((100 * 3 * 2 * k * 8 + 255) // 256 * 256 if on else 0), (n, k)


def QP(**kw):
    base = dict(T=64, d_model=48, d_out=32, dtype=_lib.PKM_BF16, reserved=0)
    base.update(kw)
    return _lib.QueryProblem(base["T"], base["d_model"], base["d_out"], base["dtype"], base["reserved"])


def test_query_struct_layout():
    assert ctypes.sizeof(_lib.QueryProblem) == 24


@pytest.mark.parametrize("kw,code", [
    (dict(d_model=12), 2), (dict(d_out=4), 2), (dict(d_model=0), 2), (dict(T=-1), 2),
    (dict(reserved=1), 2), (dict(dtype=7), 3),
])
def test_query_rejects_bad_shapes(kw, code):
    assert _lib.query_workspace_bytes(QP(**kw), False) == (1 << 64) - 1
    args = [FAKE] * 2 + [None, None]
    rc = _lib.query_forward(QP(**kw), *args, 1e-5, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, None)
    assert rc == code, _lib.STATUS.get(rc)


def test_query_argument_checks():
    qp = QP()
    need_f, need_b = _lib.query_workspace_bytes(qp, False), _lib.query_workspace_bytes(qp, True)
    assert 0 < need_f < need_b            # the backward also keeps dz [T][d_out]
    assert need_b >= 64 * 32 * 4
    fwd = lambda **o: _lib.query_forward(qp, FAKE, FAKE, o.get("g"), None, o.get("eps", 1e-5),  # noqa: E731
                                         FAKE, FAKE, FAKE, FAKE, o.get("ws", FAKE),
                                         o.get("nb", need_f), None)
    assert fwd(eps=0.0) == 7 and fwd(eps=float("nan")) == 7
    assert fwd(ws=None) == 1 and fwd(nb=need_f - 1) == 4 and fwd(ws=FAKE + 4) == 6
    assert fwd(g=FAKE + 8) == 6
    rc = _lib.query_backward(qp, FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None,
                             FAKE, need_b - 1, None)
    assert rc == 4
    rc = _lib.query_backward(qp, FAKE, FAKE, None, FAKE, FAKE, FAKE, None, FAKE, FAKE, None, None,
                             FAKE, need_b, None)
    assert rc == 1
