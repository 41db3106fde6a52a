"""The query network q = BN(x W^T) and its backward on the GPU, through the C
ABI, against oracle/query.py (float64).  Tolerances from the arithmetic:
z is a float32 sum of exact products (relative 1e-5 of the row's norm at
K <= 1600); q is z normalised and rounded once (fp32: 2e-5 relative; bf16:
half an ulp of the storage type plus 1e-4 absolute); gradients
are float32 sums, with dz split into two bfloat16 parts for bf16 storage
(~16 bits): per-row relative L2 within 1e-4 (the gate of both dtypes), and
within 2e-5 of the rms row as a tight check."""
import numpy as np
import pytest
import torch

import pkm_inputs
from gpu_util import device, to_dev, to_host
from oracle import query as Q

pytestmark = pytest.mark.gpu


def _rows_rel(got, want):
    num = np.linalg.norm(got - want, axis=-1)
    rms = np.sqrt((want ** 2).sum(axis=-1).mean())
    den = np.maximum(np.linalg.norm(want, axis=-1), 1e-3 * rms)
    return float((num / den).max()), float((num / rms).max())


def _bf16_q_ok(got_bits, want64):
    """bf16 q: within the rounding of the storage type (half an ulp, at most
    2^-8 of |q|) plus the float32 computation's absolute error (q has unit
    variance; near zero the cancellation z - mean leaves ~1e-5)."""
    got = pkm_inputs.bf16_to_f32(got_bits).astype(np.float64)
    excess = np.abs(got - want64) - 2.0 ** -8 * np.abs(want64)
    return float(excess.max()) <= 1e-4


def _run(T, dm, D, dtype, seed, affine):
    import product_key_memory_amd as pk
    dev = device()
    rng = np.random.default_rng(seed)
    x32 = rng.standard_normal((T, dm), dtype=np.float32)
    W32 = (rng.standard_normal((D, dm), dtype=np.float32) * np.float32(dm ** -0.5))
    g = (1.0 + 0.1 * rng.standard_normal(D)).astype(np.float32) if affine else None
    b = (0.1 * rng.standard_normal(D)).astype(np.float32) if affine else None
    dq = rng.standard_normal((T, D), dtype=np.float32)
    if dtype == "bf16":
        x, W = pkm_inputs.bf16_bits(x32), pkm_inputs.bf16_bits(W32)
    else:
        x, W = x32, W32
    print(f"[query] T={T} d_model={dm} d_out={D} {dtype} affine={affine}", flush=True)
    xd, Wd = to_dev(x, dev), to_dev(W, dev)
    gd = to_dev(g, dev) if affine else None
    bd = to_dev(b, dev) if affine else None
    q, z, mean, rstd = pk.pkm_query_forward(xd, Wd, gd, bd, 1e-5)
    dx, dW, dgamma, dbeta = pk.pkm_query_backward(xd, Wd, gd, z, mean, rstd, to_dev(dq, dev))
    torch.cuda.synchronize()
    ref = Q.query_forward(x, W, g, b, 1e-5)
    gref = Q.query_backward(x, W, dq, g, 1e-5)
    return (to_host(q), to_host(z), to_host(mean), to_host(rstd), to_host(dx), to_host(dW),
            to_host(dgamma), to_host(dbeta)), ref, gref


@pytest.mark.parametrize("T", [300, 301, 299])
@pytest.mark.parametrize("dtype,affine", [("fp32", False), ("fp32", True), ("bf16", True)])
def test_query_small_ragged(dtype, affine, T):
    """Sizes that leave ragged 128 x 128 tiles and a ragged 32-wide K step;
    token counts that are not multiples of 4 or 8 (the dW product runs over the
    tokens as its K)."""
    (q, z, mean, rstd, dx, dW, dg, db), ref, gref = _run(T, 72, 40, dtype, 91, affine)
    assert _rows_rel(z, ref["z"])[0] <= 1e-5
    assert np.allclose(mean, ref["mean"], rtol=1e-4, atol=1e-5)
    assert np.allclose(rstd, ref["rstd"], rtol=1e-4)
    if dtype == "bf16":
        assert _bf16_q_ok(q, ref["q"])
    else:
        assert _rows_rel(q, ref["q"])[0] <= 2e-5
    for got, want in ((dx, gref["dx"]), (dW, gref["dW"])):
        gate, tight = _rows_rel(got, want)
        assert gate <= 1e-4 and tight <= 2e-5, (gate, tight)
    assert np.allclose(dg, gref["dgamma"], rtol=1e-4, atol=1e-3)
    assert np.allclose(db, gref["dbeta"], rtol=1e-4, atol=1e-3)


@pytest.mark.parametrize("T,dm,D", [(300, 128, 64), (33, 64, 192)])
def test_query_direct_lds_path(T, dm, D):
    """bf16 with every K a multiple of 64 (d_model, d_out and the padded token
    count): all three products take the direct-to-LDS kernel, here with ragged
    row and column tiles (rows past M or N are fed from the last row and not
    stored) and, for T = 33, a single 64-wide K stage in the dW product."""
    (q, z, mean, rstd, dx, dW, dg, db), ref, gref = _run(T, dm, D, "bf16", 94, True)
    assert _rows_rel(z, ref["z"])[0] <= 1e-5
    assert _bf16_q_ok(q, ref["q"])
    for got, want in ((dx, gref["dx"]), (dW, gref["dW"])):
        gate, tight = _rows_rel(got, want)
        assert gate <= 1e-4 and tight <= 2e-5, (gate, tight)
    assert np.allclose(dg, gref["dgamma"], rtol=1e-4, atol=1e-3)
    assert np.allclose(db, gref["dbeta"], rtol=1e-4, atol=1e-3)


@pytest.mark.slow
def test_query_many_tokens():
    """More 64-token tiles than a launch's y extent allows (T = 2^22 + 37:
    65,537 tiles of the padded token pitch): the transposes and the fused
    batch-norm step walk their token tiles by the grid's y extent, and the
    products run on 1-D grids of tiles."""
    T = (1 << 22) + 37
    (q, z, mean, rstd, dx, dW, dg, db), ref, gref = _run(T, 8, 8, "bf16", 95, False)
    assert _rows_rel(z, ref["z"])[0] <= 1e-5
    assert _bf16_q_ok(q, ref["q"])
    for got, want in ((dx, gref["dx"]), (dW, gref["dW"])):
        gate, tight = _rows_rel(got, want)
        assert gate <= 1e-4 and tight <= 2e-5, (gate, tight)


@pytest.mark.slow
def test_query_model_width():
    """The workload's widths: d_model = 1600 (the pages' model), d_out = H d_k = 2048."""
    (q, z, mean, rstd, dx, dW, dg, db), ref, gref = _run(2048, 1600, 2048, "bf16", 92, True)
    assert _rows_rel(z, ref["z"])[0] <= 1e-5
    assert _bf16_q_ok(q, ref["q"])
    for got, want in ((dx, gref["dx"]), (dW, gref["dW"])):
        gate, tight = _rows_rel(got, want)
        assert gate <= 1e-4 and tight <= 2e-5, (gate, tight)


def test_query_feeds_the_layer():
    """q from the library is a valid pkm_forward input: BN statistics of every
    feature are (0, ~1) over the batch."""
    import product_key_memory_amd as pk
    dev = device()
    g = torch.Generator(device=dev).manual_seed(93)
    x = torch.randn((4096, 512), device=dev, generator=g).to(torch.bfloat16)
    W = (torch.randn((512, 512), device=dev, generator=g) * 512 ** -0.5).to(torch.bfloat16)
    q, z, mean, rstd = pk.pkm_query_forward(x, W)
    qf = q.float()
    assert qf.mean(0).abs().max().item() < 1e-2
    assert (qf.var(0, unbiased=False) - 1).abs().max().item() < 2e-2
