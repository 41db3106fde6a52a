"""pkm_backward_noalloc -- pkm_backward with the library's static scratch
instead of a caller workspace -- through the C ABI: the same dq, dkeys and
dvalues bit for bit as pkm_backward, on two calls in a row (the benchmark
workload, 113 MiB of the 128 MiB scratch, then a smaller problem: the second
call runs over what the first left in the array); a problem too large for
the array is rejected on the host before anything is enqueued."""
import pytest
import torch

import gpu_util
import pkm_inputs
from product_key_memory_amd import _lib

FAKE = 1 << 20          # an aligned address the rejected call never touches


def _against_backward(inp, k):
    import product_key_memory_amd as pk
    dev = gpu_util.device()
    w = inp["w"]
    print(f"[noalloc] {w.name} T={w.T} H={w.H} n={w.n} k={k} d_v={w.d_v} {w.dtype}", flush=True)
    q, keys, values, dy = (gpu_util.to_dev(inp[x], dev) for x in ("q", "keys", "values", "dy"))
    _, idx, wts, _ = pk.pkm_forward(q, keys, values, k)
    start = torch.randn((w.n * w.n, w.d_v), dtype=torch.float32, device=dev)
    dv_ref = start.clone()
    dq_ref, dk_ref, _ = pk.pkm_backward(q, keys, values, idx, wts, dy, dvalues=dv_ref)
    dq = torch.full_like(dq_ref, float("nan"))
    dk = torch.full_like(dk_ref, float("nan"))
    dv = start.clone()
    p = pk.problem(w.T, w.H, w.n, k, w.d_k, w.d_v, q.dtype)
    rc = _lib.backward_noalloc(p, q.data_ptr(), keys.data_ptr(), values.data_ptr(),
                               idx.data_ptr(), wts.data_ptr(), dy.data_ptr(), dq.data_ptr(),
                               dk.data_ptr(), dv.data_ptr(),
                               torch.cuda.current_stream(dev).cuda_stream)
    assert rc == 0, _lib.STATUS.get(rc)
    torch.cuda.synchronize()
    assert torch.equal(dq, dq_ref), "dq differs from pkm_backward"
    assert torch.equal(dk, dk_ref), "dkeys differs from pkm_backward"
    assert torch.equal(dv, dv_ref), "dvalues differs from pkm_backward"


@pytest.mark.gpu
def test_noalloc_matches_backward_on_two_calls():
    _against_backward(pkm_inputs.make("base-bf16-zipf-bwd"), 32)
    _against_backward(pkm_inputs.custom(300, 2, 40, 8, 32, 64, dtype="bf16", seed=901), 8)


def test_noalloc_rejects_a_problem_beyond_its_scratch():
    # 16384 tokens, 8 heads, 1024^2 slots, k = 32, d_v = 1600: 164 MiB > 128 MiB
    p = _lib.Problem(16384, 8, 1024, 32, 512, 1600, _lib.PKM_BF16)
    assert _lib.workspace_bytes(p, 1) > 128 << 20
    assert _lib.backward_noalloc(p, *[FAKE] * 9, None) == 8
    ok = _lib.Problem(16384, 4, 512, 32, 512, 1024, _lib.PKM_BF16)
    assert _lib.workspace_bytes(ok, 1) <= 128 << 20
