"""The sparse value update (SGD, lazy Adam) and the slot-usage counter on the
GPU, through the C ABI, against oracle/update.py.  Usage is integer work:
bit-exact.  Updated values: within one unit in the last place of the storage
type (the oracle rounds float64 -> float32 -> storage, the GPU its float32
fused result once; they differ only on double-rounding ties), rows no pick
selected bit-identical to the input.  Adam moments: float32 sums against
float64, relative 1e-5 of the row's largest moment; Adam values (float32
storage): within 1e-5 * lr absolute, since the float32 step itself carries a
few roundings."""
import numpy as np
import pytest
import torch

import pkm_inputs
from gpu_util import device, to_dev, to_host
from oracle import update as U

pytestmark = pytest.mark.gpu


def _ulp_diff(a: np.ndarray, b: np.ndarray) -> int:
    if a.dtype == np.uint16:
        return int(np.abs(a.astype(np.int64) - b.astype(np.int64)).max())
    ia = a.view(np.int32).astype(np.int64)
    ib = b.view(np.int32).astype(np.int64)
    return int(np.abs(ia - ib).max())


def _setup(n, d_v, dtype, T, H, k, seed):
    rng = np.random.default_rng(seed)
    vals32 = rng.standard_normal((n * n, d_v), dtype=np.float32) * np.float32(0.05)
    vals = pkm_inputs.bf16_bits(vals32) if dtype == "bf16" else vals32
    grads = rng.standard_normal((n * n, d_v), dtype=np.float32)
    idx = pkm_inputs.zipf_slots(rng, T * H * k, n * n, 1.1).reshape(T, H, k)
    return vals, grads, idx


def _sort(idx, n, dev):
    import product_key_memory_amd as pk
    slot_start, _ = pk.pkm_slot_sort(to_dev(idx.astype(np.int32), dev), n)
    return slot_start


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_sparse_sgd(dtype):
    import product_key_memory_amd as pk
    dev = device()
    n, d_v = 64, 40
    vals, grads, idx = _setup(n, d_v, dtype, T=300, H=2, k=8, seed=81)
    print(f"[update] sgd n={n} d_v={d_v} {dtype}", flush=True)
    slot_start = _sort(idx, n, dev)
    v_dev = to_dev(vals, dev)
    pk.pkm_sparse_sgd(v_dev, to_dev(grads, dev), slot_start, 0.03)
    got = to_host(v_dev)
    touched = U.touched_slots([idx], n)
    want = U.sparse_sgd(vals, grads, touched, 0.03)
    assert np.array_equal(got[~touched], vals[~touched])
    assert _ulp_diff(got[touched], want[touched]) <= 1
    assert (got[touched] == want[touched]).mean() > 0.999


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_sparse_adam_three_steps(dtype):
    """Three steps, a new batch each: rows selected at some steps only keep
    their moments in between."""
    import product_key_memory_amd as pk
    dev = device()
    n, d_v = 32, 24
    vals, _, _ = _setup(n, d_v, dtype, T=1, H=1, k=1, seed=82)
    rng = np.random.default_rng(83)
    v_dev = to_dev(vals, dev)
    m_dev = torch.zeros((n * n, d_v), dtype=torch.float32, device=dev)
    s_dev = torch.zeros_like(m_dev)
    ref_v, ref_m, ref_s = vals.copy(), np.zeros((n * n, d_v), np.float32), np.zeros((n * n, d_v), np.float32)
    for step in (1, 2, 3):
        idx = rng.integers(0, n * n, size=(50, 2, 4))
        grads = rng.standard_normal((n * n, d_v), dtype=np.float32)
        print(f"[update] adam step {step} {dtype}", flush=True)
        slot_start = _sort(idx, n, dev)
        pk.pkm_sparse_adam(v_dev, to_dev(grads, dev), slot_start, m_dev, s_dev, step, 0.01)
        touched = U.touched_slots([idx], n)
        ref_v, ref_m, ref_s = U.sparse_adam(ref_v, grads, touched, ref_m, ref_s, step, 0.01,
                                            0.9, 0.999, 1e-8)
        got_v, got_m, got_s = to_host(v_dev), to_host(m_dev), to_host(s_dev)
        for got, want in ((got_m, ref_m), (got_s, ref_s)):
            scale = np.maximum(np.abs(want).max(axis=1, keepdims=True), 1e-30)
            assert (np.abs(got - want) / scale).max() <= 1e-5
        # values: the float32 step (m/c1)/(sqrt(v/c2)+eps), about 1 in size,
        # carries a few float32 roundings, so w - lr*step is off by about
        # lr * 1e-7 in absolute terms (many ulps where w - lr*step nearly
        # cancels); bf16 storage rounds that away except at ties
        if dtype == "fp32":
            assert np.abs(got_v - ref_v).max() <= 1e-5 * 0.01
        else:
            assert _ulp_diff(got_v, ref_v) <= 1


def test_slot_usage_two_batches():
    import product_key_memory_amd as pk
    dev = device()
    n = 512
    rng = np.random.default_rng(84)
    b1 = pkm_inputs.zipf_slots(rng, 16384 * 4 * 32, n * n, 1.1).reshape(16384, 4, 32)
    b2 = rng.integers(0, n * n, size=(3001, 2, 7))
    print("[update] usage", flush=True)
    counts, used = pk.pkm_slot_usage(_sort(b1, n, dev))
    want, want_used = U.slot_usage([b1], n)
    assert np.array_equal(to_host(counts), want) and int(to_host(used)[0]) == want_used
    counts, used = pk.pkm_slot_usage(_sort(b2, n, dev), counts)
    want, want_used = U.slot_usage([b1, b2], n)
    assert np.array_equal(to_host(counts), want) and int(to_host(used)[0]) == want_used


def test_sparse_sgd_bench_size_sampled():
    """512^2 slots x 1024 bf16 (the benchmark's table): sampled rows."""
    import product_key_memory_amd as pk
    dev = device()
    n, d_v = 512, 1024
    rng = np.random.default_rng(85)
    idx = pkm_inputs.zipf_slots(rng, 16384 * 4 * 32, n * n, 1.1).reshape(16384, 4, 32)
    print("[update] sgd bench size", flush=True)
    v_dev = torch.randn((n * n, d_v), device=dev, generator=torch.Generator(device=dev).manual_seed(86)).to(torch.bfloat16)
    g_dev = torch.randn((n * n, d_v), device=dev, generator=torch.Generator(device=dev).manual_seed(87))
    before = v_dev.clone()
    pk.pkm_sparse_sgd(v_dev, g_dev, _sort(idx, n, dev), 0.05)
    touched = U.touched_slots([idx], n)
    rows = np.concatenate([rng.choice(np.nonzero(touched)[0], 2000, replace=False),
                           rng.choice(np.nonzero(~touched)[0], 200, replace=False)])
    rows_t = torch.from_numpy(rows).to(dev)
    vals = to_host(before[rows_t].contiguous())
    want = U.sparse_sgd(vals, to_host(g_dev[rows_t].contiguous()), touched[rows], 0.05)
    got = to_host(v_dev[rows_t].contiguous())
    assert np.array_equal(got[~touched[rows]], vals[~touched[rows]])
    assert _ulp_diff(got, want) <= 1
