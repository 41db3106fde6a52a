"""GPU path (through the C ABI) against the CPU oracle, element by element.

Every test prints the case it runs before touching the GPU.  Rules and
tolerances are in parity.py.
"""
import numpy as np
import pytest
import torch

import gpu_util
import pkm_inputs

pytestmark = pytest.mark.gpu

# Besides the gate tolerances, the errors expected from the arithmetic itself:
# float32 accumulation everywhere, and for bf16 one rounding of y on store
# (y: per-row relative error; gradients: error relative to the rms row norm).
TIGHT = {"fp32": {"y": 5e-5, "grad": 2e-5}, "bf16": {"y": 6e-3, "grad": 5e-5}}


def test_tiny_fp32_full(orc):
    inp = pkm_inputs.make("tiny-fp32", with_dy=True)
    gpu_util.run_parity(orc, inp, inp["w"].k, backward=True, tight=TIGHT["fp32"])


def test_proj_fp32_full(orc):
    inp = pkm_inputs.make("proj-fp32", with_dy=True)
    gpu_util.run_parity(orc, inp, inp["w"].k, backward=True, tight=TIGHT["fp32"])


def test_base_bf16_sampled(orc):
    inp = pkm_inputs.make("base-bf16")
    sub = pkm_inputs.token_subset(inp["w"].T, 1024, seed=7)
    gpu_util.run_parity(orc, inp, inp["w"].k, subset=sub, tight=TIGHT["bf16"])


def test_base_bf16_zipf_bwd_sampled(orc):
    inp = pkm_inputs.make("base-bf16-zipf-bwd")
    sub = pkm_inputs.token_subset(inp["w"].T, 1024, seed=8)
    gpu_util.run_parity(orc, inp, inp["w"].k, subset=sub, backward=True, tight=TIGHT["bf16"])


def test_base_bf16_zipf_bwd_invariants():
    """Full-size backward invariants (no oracle): column sums of dvalues equal
    H * sum_t dy[t] (the weights of a head sum to 1), unselected rows stay 0."""
    import product_key_memory_amd as pk
    dev = gpu_util.device()
    inp = pkm_inputs.make("base-bf16-zipf-bwd")
    w = inp["w"]
    print(f"[invariants] {w.name}", flush=True)
    q, keys, values, dy = (gpu_util.to_dev(inp[x], dev) for x in ("q", "keys", "values", "dy"))
    y, idx, wts, _ = pk.pkm_forward(q, keys, values, w.k)
    assert torch.allclose(wts.sum(dim=2), torch.ones_like(wts[:, :, 0]), atol=1e-5)
    dq, dkeys, dvalues = pk.pkm_backward(q, keys, values, idx, wts, dy)
    torch.cuda.synchronize()
    col = dvalues.double().sum(dim=0)
    want = w.H * dy.double().sum(dim=0)
    scale = w.H * dy.double().abs().sum(dim=0)
    assert torch.all((col - want).abs() <= 1e-5 * scale + 1e-6), "dvalues column sums"
    touched = torch.zeros(w.slots, dtype=torch.bool, device=dev)
    touched[idx.reshape(-1).long()] = True
    assert torch.all(dvalues[~touched] == 0), "unselected rows must stay exactly 0"
    # hot slots from the Zipf bias: report the top-1 hit histogram head
    top1 = idx[:, :, 0].reshape(-1).long()
    counts = torch.bincount(top1, minlength=w.slots).sort(descending=True).values[:5]
    print(f"[invariants] top-1 hits of the 5 hottest slots: {counts.tolist()} of {top1.numel()}")


@pytest.mark.slow
def test_large_bf16_zipf_bwd_sampled(orc):
    inp = pkm_inputs.make("large-bf16-zipf-bwd")
    sub = pkm_inputs.token_subset(inp["w"].T, 256, seed=9)
    gpu_util.run_parity(orc, inp, inp["w"].k, subset=sub, backward=True, tight=TIGHT["bf16"])


# ---------------------------------------------------------------------------
# edge cases: small problems, checked in full
# ---------------------------------------------------------------------------
EDGE = [
    # T,  H, n,   k,  d_k,  d_v,  kind
    (37, 3, 37, 5, 48, 24, "normal"),        # ragged T, n not a multiple of 16, partial MFMA K step
    (33, 1, 64, 64, 32, 8, "normal"),        # k = n = 64 (largest k), one 16-byte value chunk
    (20, 2, 32, 32, 16, 16, "normal"),       # k = n, smallest d_k
    (50, 2, 16, 1, 64, 40, "normal"),        # k = 1
    (9, 1, 1, 1, 16, 8, "normal"),           # one slot
    (40, 2, 24, 6, 32, 16, "integer"),       # exact arithmetic: exact ties everywhere
    (40, 2, 20, 7, 32, 16, "dup"),           # duplicated sub-keys
    (24, 1, 96, 9, 32, 16, "right_zero"),    # every right score ties: all n survive the filter
    (12, 2, 1024, 32, 64, 16, "right_zero"), # all 1024 survive: the widest sort
    (18, 2, 130, 17, 1024, 1600, "normal"),  # widest d_k, ragged value row
    (6, 1, 8, 3, 16, 4096, "normal"),        # widest backward row
    (70, 8, 40, 12, 32, 64, "normal"),       # many heads
]


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("case", EDGE, ids=[f"T{c[0]}H{c[1]}n{c[2]}k{c[3]}dk{c[4]}dv{c[5]}-{c[6]}" for c in EDGE])
def test_edge(orc, case, dtype):
    T, H, n, k, d_k, d_v, kind = case
    inp = pkm_inputs.custom(T, H, n, k, d_k, d_v, dtype=dtype, seed=T * 131 + n, kind=kind)
    rep = gpu_util.run_parity(orc, inp, k, backward=True, tight=TIGHT[dtype])
    if kind in ("integer", "right_zero") and dtype == "fp32":
        # exact float32 arithmetic: the order itself, ties included, is the oracle's
        import product_key_memory_amd as pk
        dev = gpu_util.device()
        q, keys, values = (gpu_util.to_dev(inp[x], dev) for x in ("q", "keys", "values"))
        _, idx, _, _ = pk.pkm_forward(q, keys, values, k)
        ref = orc.forward(inp["q"], inp["keys"], inp["values"], k)
        assert np.array_equal(gpu_util.to_host(idx), ref["idx"]), "exact-arithmetic order differs"
    assert rep["rows"] == T * H


# the two-kernel selection (d_k = 512, k <= 32; bf16 with 128 <= n <= 1024,
# float32 with 128 <= n <= 256): per-half top-k over blocks of 128, 256 or 512
# sub-keys, then the pruned combine
FAST_EDGE = [
    (50, 2, 128, 16, 512, 16, "normal"),      # smallest n on the path: 256-sub-key blocks, groups of 4
    (37, 3, 200, 32, 512, 24, "dup"),         # ragged n in a 256-block, duplicated sub-keys
    (20, 1, 256, 32, 512, 16, "right_zero"),  # all right scores tie in a 256-block: exact bisection
    (33, 2, 130, 7, 512, 16, "integer"),      # exact arithmetic in a 256-block
    # T,  H, n,    k,  d_k, d_v, kind
    (100, 3, 300, 20, 512, 24, "normal"),      # ragged T and n, k < 32
    (70, 2, 257, 32, 512, 16, "normal"),       # smallest n on the path: one sub-key in the last tile
    (64, 2, 512, 1, 512, 16, "normal"),        # k = 1
    (48, 2, 400, 32, 512, 16, "dup"),          # duplicated sub-keys
    (30, 1, 512, 32, 512, 16, "right_zero"),   # every right score ties: the exact bisection branch
    (40, 2, 300, 9, 512, 16, "integer"),       # exact arithmetic, ties everywhere
    (24, 2, 1024, 32, 512, 16, "normal"),      # two full blocks
    (40, 2, 600, 32, 512, 16, "normal"),       # a second block of 88 sub-keys
    (40, 1, 520, 32, 512, 16, "normal"),       # a second block with fewer sub-keys than k
    (24, 2, 1024, 32, 512, 16, "dup"),         # ties across the blocks (sub-key 0 = sub-key n-1)
    (12, 1, 1024, 32, 512, 16, "right_zero"),  # the exact branch in both blocks
    (30, 2, 700, 5, 512, 16, "integer"),       # exact arithmetic across the blocks
]
FAST_EDGE = [c + ("bf16",) for c in FAST_EDGE] + [
    # float32 storage, scored on the fp64 MFMA in blocks of 128 sub-keys
    (50, 2, 128, 16, 512, 16, "normal", "fp32"),      # one block
    (37, 3, 200, 32, 512, 24, "dup", "fp32"),         # two blocks, duplicated sub-keys
    (40, 2, 129, 32, 512, 16, "normal", "fp32"),      # a second block of one sub-key (< k)
    (20, 1, 256, 32, 512, 16, "right_zero", "fp32"),  # the exact bisection in both blocks
    (33, 2, 130, 7, 512, 16, "integer", "fp32"),      # exact arithmetic: the oracle's order
]


@pytest.mark.parametrize("case", FAST_EDGE,
                         ids=[f"T{c[0]}H{c[1]}n{c[2]}k{c[3]}-{c[6]}-{c[7]}" for c in FAST_EDGE])
def test_edge_two_kernel_selection(orc, case):
    import product_key_memory_amd as pk
    from product_key_memory_amd import _lib
    T, H, n, k, d_k, d_v, kind, dtype = case
    code = _lib.PKM_BF16 if dtype == "bf16" else _lib.PKM_FP32
    # this shape takes the two-kernel path: it is the one that needs a forward workspace
    assert _lib.workspace_bytes(_lib.Problem(T, H, n, k, d_k, d_v, code), False) > 0
    inp = pkm_inputs.custom(T, H, n, k, d_k, d_v, dtype=dtype, seed=T * 131 + n + 7, kind=kind)
    rep = gpu_util.run_parity(orc, inp, k, backward=True, tight=TIGHT[dtype])
    assert rep["rows"] == T * H
    if kind == "integer" or (kind == "right_zero" and dtype == "fp32"):
        # exact arithmetic: the order itself, ties included, is the oracle's
        dev = gpu_util.device()
        q, keys, values = (gpu_util.to_dev(inp[x], dev) for x in ("q", "keys", "values"))
        _, idx, _, _ = pk.pkm_forward(q, keys, values, k)
        ref = orc.forward(inp["q"], inp["keys"], inp["values"], k)
        assert np.array_equal(gpu_util.to_host(idx), ref["idx"]), "exact-arithmetic order differs"


# T not a multiple of 64 leaves tokens past T in the last workgroup; those
# lanes score token 0's query.  With token 0's query zero, every sub-key ties
# (more than 64 survivors in both halves): the lanes past T must keep nothing,
# also in waves whose live tokens need no bisection and in waves with no live
# token at all, and must not disturb the live tokens' survivors.
TAIL_CASES = [(65, 512, "bf16"), (100, 512, "bf16"), (112, 512, "bf16"), (100, 1024, "bf16"),
              (100, 200, "bf16"), (100, 200, "fp32")]


@pytest.mark.parametrize("T,n,dtype", TAIL_CASES, ids=[f"T{c[0]}n{c[1]}-{c[2]}" for c in TAIL_CASES])
def test_two_kernel_selection_tail_tokens_with_tied_token0(orc, T, n, dtype):
    from product_key_memory_amd import _lib
    code = _lib.PKM_BF16 if dtype == "bf16" else _lib.PKM_FP32
    assert _lib.workspace_bytes(_lib.Problem(T, 2, n, 32, 512, 16, code), False) > 0
    inp = pkm_inputs.custom(T, 2, n, 32, 512, 16, dtype=dtype, seed=T + n)
    inp["q"][0] = 0          # +0: every score of token 0 is exactly 0
    rep = gpu_util.run_parity(orc, inp, 32, tight=TIGHT[dtype])
    assert rep["rows"] == T * 2


def test_k1_is_the_row_itself(orc):
    """k = 1, one head: the weight is exactly 1 and y is the selected value row, bit for bit."""
    import product_key_memory_amd as pk
    dev = gpu_util.device()
    inp = pkm_inputs.custom(64, 1, 48, 1, 32, 64, dtype="fp32", seed=5)
    q, keys, values = (gpu_util.to_dev(inp[x], dev) for x in ("q", "keys", "values"))
    y, idx, wts, _ = pk.pkm_forward(q, keys, values, 1)
    ref = orc.forward(inp["q"], inp["keys"], inp["values"], 1)
    g_idx = gpu_util.to_host(idx)
    assert np.array_equal(g_idx, ref["idx"])
    assert np.all(gpu_util.to_host(wts) == 1.0)
    assert np.array_equal(gpu_util.to_host(y), inp["values"][g_idx[:, 0, 0]])


def test_empty_batch_is_a_noop():
    import product_key_memory_amd as pk
    dev = gpu_util.device()
    q = torch.zeros((0, 2, 32), device=dev)
    keys = torch.randn((2, 2, 8, 16), device=dev)
    values = torch.randn((64, 8), device=dev)
    y, idx, wts, sc = pk.pkm_forward(q, keys, values, 4)
    assert y.shape == (0, 8) and idx.shape == (0, 2, 4)
    dq, dkeys, dvalues = pk.pkm_backward(q, keys, values, idx, wts, torch.zeros((0, 8), device=dev))
    torch.cuda.synchronize()
    assert torch.all(dkeys == 0) and torch.all(dvalues == 0)


def test_autograd_function(orc):
    """ProductKeyMemoryFunction wires the library's backward into autograd."""
    import product_key_memory_amd as pk
    dev = gpu_util.device()
    inp = pkm_inputs.custom(32, 2, 16, 4, 32, 16, dtype="fp32", seed=3)
    q, keys, values = (gpu_util.to_dev(inp[x], dev).requires_grad_() for x in ("q", "keys", "values"))
    y = pk.ProductKeyMemoryFunction.apply(q, keys, values, 4)
    dy = gpu_util.to_dev(inp["dy"], dev)
    (y * dy).sum().backward()
    ref = orc.forward(inp["q"], inp["keys"], inp["values"], 4)
    ob = orc.backward(inp["q"], inp["keys"], inp["values"], ref["idx"], ref["weights"], inp["dy"])
    assert np.allclose(q.grad.cpu().numpy(), ob["dq"], rtol=1e-4, atol=1e-5)
    assert np.allclose(keys.grad.cpu().numpy(), ob["dkeys"], rtol=1e-4, atol=1e-5)
    assert np.allclose(values.grad.cpu().numpy(), ob["dvalues"], rtol=1e-4, atol=1e-5)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_dvalues_accumulate_mode(orc, dtype):
    """A given dvalues is accumulated into: result - prefill equals the
    overwrite-mode gradient (same kernels, same sums), rows nobody picked keep
    the prefill bit for bit."""
    import product_key_memory_amd as pk
    dev = gpu_util.device()
    inp = pkm_inputs.custom(300, 2, 40, 8, 32, 64, dtype=dtype, seed=77)
    print(f"[accumulate] {dtype}", flush=True)
    q, keys, values, dy = (gpu_util.to_dev(inp[x], dev) for x in ("q", "keys", "values", "dy"))
    _, idx, wts, _ = pk.pkm_forward(q, keys, values, 8)
    _, _, fresh = pk.pkm_backward(q, keys, values, idx, wts, dy)
    prefill = torch.randn((40 * 40, 64), device=dev)
    acc = prefill.clone()
    pk.pkm_backward(q, keys, values, idx, wts, dy, dvalues=acc)
    torch.cuda.synchronize()
    touched = torch.zeros(1600, dtype=torch.bool, device=dev)
    touched[idx.reshape(-1).long()] = True
    assert torch.equal(acc[~touched], prefill[~touched])
    assert torch.all(fresh[~touched] == 0)
    diff = (acc - prefill)[touched].double()
    ref = fresh[touched].double()
    assert torch.allclose(diff, ref, rtol=1e-5, atol=1e-6 * ref.abs().max().item())
