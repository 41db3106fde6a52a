"""The slot sort (pkm_slot_sort) against its plain definition: slot_start is
the exclusive prefix sum of the per-slot pick counts, and order lists, slot by
slot, exactly the picks that chose that slot, in ascending pick id -- the
stable argsort of the flat idx.  Index work, so bit-exact."""
import numpy as np
import pytest

import pkm_inputs
from gpu_util import device, to_dev, to_host

pytestmark = pytest.mark.gpu


def _expected(idx: np.ndarray, n: int):
    flat = idx.reshape(-1).astype(np.int64)
    counts = np.bincount(flat, minlength=n * n)
    start = np.zeros(n * n + 1, dtype=np.int64)
    np.cumsum(counts, out=start[1:])
    return start, np.argsort(flat, kind="stable")


def _check(idx: np.ndarray, n: int):
    import product_key_memory_amd as pk

    dev = device()
    print(f"[slot_sort] idx {idx.shape} n={n}", flush=True)
    g_start, g_order = pk.pkm_slot_sort(to_dev(idx.astype(np.int32), dev), n)
    g_start, g_order = to_host(g_start).astype(np.int64), to_host(g_order).astype(np.int64)
    start, order = _expected(idx, n)
    np.testing.assert_array_equal(g_start, start)
    np.testing.assert_array_equal(g_order, order)


def test_slot_sort_zipf_base():
    """512^2 slots, 16384 x 4 x 32 picks drawn Zipf(1.1) over the slots (hot rows)."""
    rng = np.random.default_rng(71)
    idx = pkm_inputs.zipf_slots(rng, 16384 * 4 * 32, 512 * 512, 1.1).reshape(16384, 4, 32)
    _check(idx, 512)


def test_slot_sort_uniform_ragged():
    """1000^2 slots (not a power of two), a ragged pick count."""
    rng = np.random.default_rng(72)
    idx = rng.integers(0, 1000 * 1000, size=(3001, 2, 7))
    _check(idx, 1000)


@pytest.mark.parametrize("n,T,H,k", [(32, 5, 1, 3), (4, 3, 1, 4), (17, 1000, 3, 5)])
def test_slot_sort_small(n, T, H, k):
    rng = np.random.default_rng(73 + n)
    _check(rng.integers(0, n * n, size=(T, H, k)), n)


def test_slot_sort_one_hot_slot():
    """Every pick in the last slot: one bucket holds all picks."""
    idx = np.full((4096, 1, 16), 64 * 64 - 1, dtype=np.int64)
    _check(idx, 64)


def test_slot_sort_two_keys_interleaved():
    """Picks alternating between two slots of one bucket and a slot of another,
    in every lane pattern: the stable placement inside waves and across the
    waves of a round."""
    rng = np.random.default_rng(75)
    idx = np.where(rng.random((5000, 2, 8)) < 0.5, 7, 9)
    idx[rng.random(idx.shape) < 0.1] = 40 * 40 - 1
    _check(idx, 40)


def test_slot_sort_large_memory():
    """1024^2 slots, 16384 x 8 x 32 picks, Zipf."""
    rng = np.random.default_rng(74)
    idx = pkm_inputs.zipf_slots(rng, 16384 * 8 * 32, 1024 * 1024, 1.1).reshape(16384, 8, 32)
    _check(idx, 1024)
