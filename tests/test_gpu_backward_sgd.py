"""The backward with the SGD step fused in (pkm_backward_sgd), through the C
ABI.  Against the unfused chain, pkm_backward_overwrite followed by
pkm_sparse_sgd: the same dq, dkeys and updated values bit for bit -- both
paths sum a row's picks in ascending pick id and a long run's pieces in the
same fixed order, then apply one fused multiply-add rounded once -- and rows
no pick selected unchanged.  Against the oracle: its float64 backward and
oracle/update.py's SGD on the touched rows, within the gradient tolerance
scaled by lr."""
import numpy as np
import pytest
import torch

import pkm_inputs
from gpu_util import device, to_dev, to_host
from oracle import update as U

pytestmark = pytest.mark.gpu


def _widen(a: np.ndarray) -> np.ndarray:
    return (a.astype(np.uint32) << 16).view(np.float32) if a.dtype == np.uint16 else a


def _fused_vs_chain(inp, k, lr):
    import product_key_memory_amd as pk
    dev = device()
    w = inp["w"]
    q, keys, values, dy = (to_dev(inp[x], dev) for x in ("q", "keys", "values", "dy"))
    _, idx, wts, _ = pk.pkm_forward(q, keys, values, k)
    # the chain
    dq, dkeys, dvalues = pk.pkm_backward(q, keys, values, idx, wts, dy)
    slot_start, _ = pk.pkm_slot_sort(idx, w.n)
    v_chain = values.clone()
    pk.pkm_sparse_sgd(v_chain, dvalues, slot_start, lr)
    # fused
    v_fused = values.clone()
    dq_f, dkeys_f = pk.pkm_backward_sgd(q, keys, v_fused, idx, wts, dy, lr)
    torch.cuda.synchronize()
    assert torch.equal(dq_f, dq), "dq differs from pkm_backward"
    assert torch.equal(dkeys_f, dkeys), "dkeys differs from pkm_backward"
    counts = (slot_start[1:] - slot_start[:-1]).cpu().numpy()
    v0, vc, vf = to_host(values), to_host(v_chain), to_host(v_fused)
    untouched = counts == 0
    assert np.array_equal(vf[untouched], v0[untouched]), "unselected rows changed"
    assert np.array_equal(vf, vc), "fused update differs from backward + sparse SGD"
    return idx, wts, vf, counts


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_fused_sgd_small_against_chain_and_oracle(orc, dtype):
    inp = pkm_inputs.custom(300, 2, 40, 8, 32, 64, dtype=dtype, seed=601)
    print(f"[backward_sgd] small {dtype}", flush=True)
    lr = 0.05
    idx, wts, v_fused, counts = _fused_vs_chain(inp, 8, lr)
    ref = orc.backward(inp["q"], inp["keys"], inp["values"], to_host(idx), to_host(wts), inp["dy"])
    touched = counts > 0
    want = U.sparse_sgd(inp["values"], ref["dvalues"].astype(np.float32), touched, lr)
    got = _widen(v_fused[touched]).astype(np.float64)
    exp = _widen(want[touched]).astype(np.float64)
    # the float32 gradient rows against float64 (relative 1e-5 of the row
    # scale), times lr, plus one rounding of the storage type
    scale = np.abs(_widen(inp["values"][touched]).astype(np.float64)).max(axis=1, keepdims=True) + \
        lr * np.abs(ref["dvalues"][touched]).max(axis=1, keepdims=True)
    half_ulp = 2.0 ** -8 if dtype == "bf16" else 2.0 ** -23
    assert np.all(np.abs(got - exp) <= 2 * half_ulp * scale + 1e-5 * lr * scale)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_fused_sgd_hot_slots(dtype):
    """Every token asks the same query: each selected slot gets T*H picks, runs
    longer than one wave's share (32 picks at this batch size), so the
    long-run path carries the update."""
    inp = pkm_inputs.custom(700, 1, 24, 4, 32, 48, dtype=dtype, seed=602)
    inp["q"][:] = inp["q"][0]
    print(f"[backward_sgd] hot slots {dtype}", flush=True)
    _, _, _, counts = _fused_vs_chain(inp, 4, 0.01)
    assert (counts > 256).sum() == 4


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_fused_sgd_widest_rows(dtype):
    """d_v = 4096, the backward's widest value row (the most chunks per lane)."""
    inp = pkm_inputs.custom(64, 1, 8, 3, 16, 4096, dtype=dtype, seed=604)
    print(f"[backward_sgd] d_v 4096 {dtype}", flush=True)
    _fused_vs_chain(inp, 3, 0.02)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_fused_sgd_ragged_rows(dtype):
    """d_v = 1600 (the 1024^2-slot workload's rows): 200 16-byte chunks of bf16,
    a ragged last round of lanes, with runs long enough to take the split path."""
    inp = pkm_inputs.custom(400, 2, 12, 6, 32, 1600, dtype=dtype, seed=605)
    print(f"[backward_sgd] d_v 1600 {dtype}", flush=True)
    _fused_vs_chain(inp, 6, 0.02)


def test_fused_sgd_bench_workload():
    """The full bench workload (Zipf-hot slots: some runs are long)."""
    inp = pkm_inputs.make("base-bf16-zipf-bwd")
    print("[backward_sgd] base-bf16-zipf-bwd", flush=True)
    _, _, _, counts = _fused_vs_chain(inp, inp["w"].k, 0.01)
    assert (counts > 256).any()


def test_fused_sgd_argument_checks():
    import product_key_memory_amd as pk
    from product_key_memory_amd import _lib
    dev = device()
    inp = pkm_inputs.custom(20, 1, 16, 4, 32, 16, dtype="fp32", seed=603)
    q, keys, values, dy = (to_dev(inp[x], dev) for x in ("q", "keys", "values", "dy"))
    _, idx, wts, _ = pk.pkm_forward(q, keys, values, 4)
    with pytest.raises(pk.PKMError):
        pk.pkm_backward_sgd(q, keys, values, idx, wts, dy, float("nan"))
    p = _lib.Problem(20, 1, 16, 4, 32, 16, _lib.PKM_FP32)
    assert _lib.workspace_bytes(p, 2) >= _lib.workspace_bytes(p, 1)
    assert _lib.workspace_bytes(p, 3) == (1 << 64) - 1
