"""The flat-key search (pkm_flat_forward_select): every implied key scored
with one d_k-wide dot product, exact top-k.  Against the oracle -- itself a
flat search in float64 -- by the parity rules of every forward test
(selection sets bit-exact where the k-th / (k+1)-th gap exceeds 1e-4, weights
element-wise, y per row and element), and against the product-key selection
on the same inputs (the two searches are exact, so their sets agree wherever
the gap is clear)."""
import numpy as np
import pytest
import torch

import gpu_util
import parity
import pkm_inputs

pytestmark = pytest.mark.gpu


def _flat_parity(orc, inp, k, sub=None):
    import product_key_memory_amd as pk
    dev = gpu_util.device()
    w = inp["w"]
    qn = inp["q"] if sub is None else np.ascontiguousarray(inp["q"][sub])
    print(f"[flat] {w.name} T={qn.shape[0]} H={w.H} n={w.n} k={k}", flush=True)
    q, keys, values = gpu_util.to_dev(qn, dev), gpu_util.to_dev(inp["keys"], dev), \
        gpu_util.to_dev(inp["values"], dev)
    y, idx, wts, sc = pk.pkm_flat_forward(q, keys, values, k)
    _, idx_p, _, _ = pk.pkm_forward(q, keys, values, k)
    torch.cuda.synchronize()
    g_idx, g_w, g_sc = gpu_util.to_host(idx), gpu_util.to_host(wts), gpu_util.to_host(sc)
    ref = orc.forward(qn, inp["keys"], inp["values"], k)
    given = orc.forward_given_idx(qn, inp["keys"], inp["values"], g_idx)
    rep = parity.check_selection(g_idx, ref, given, w.n)
    assert float(np.abs(g_w - given["weights"]).max()) <= 1e-4
    serr = float((np.abs(g_sc - given["scores"]) / np.maximum(1.0, np.abs(given["scores"]))).max())
    assert serr <= 1e-4, serr
    g_y = gpu_util.bits_to_f64(gpu_util.to_host(y))
    tol = parity.TOL[w.dtype]
    parity.assert_rows_close("y", g_y, given["y"], tol)
    parity.assert_elems_close("y", g_y, given["y"], tol)
    # the product-key search reaches the same set wherever the gap is clear
    gap = parity.rel_gap(ref["kth"], ref["kth1"])
    same = np.all(np.sort(g_idx, axis=2) == np.sort(gpu_util.to_host(idx_p), axis=2), axis=2)
    assert np.all(same | (gap <= parity.GAP)), "flat and product-key sets differ above the gap"
    print(f"[flat] ok {rep}", flush=True)
    return rep


def test_flat_projection_shapes_bf16(orc):
    """The projection workload's shapes -- 4096 tokens, n = 128 (16,384 keys),
    k = 16, d_k = 512 -- in bf16 storage (the flat kernel's type), all tokens."""
    import dataclasses
    w = dataclasses.replace(pkm_inputs.WORKLOADS["proj-fp32"], dtype="bf16", name="proj-bf16")
    inp = pkm_inputs.make(w)
    _flat_parity(orc, inp, 16)


def test_flat_base_sampled(orc):
    """512^2 keys, 4 heads, k = 32: 256 seeded tokens of the base workload."""
    inp = pkm_inputs.make("base-bf16")
    _flat_parity(orc, inp, 32, sub=pkm_inputs.token_subset(inp["w"].T, 256, seed=17))


FLAT_EDGE = [
    # T, H, n, k, kind
    (37, 2, 33, 5, "normal"),        # ragged T, N = 1089: a last block of 65 keys
    (20, 1, 64, 32, "integer"),      # exact arithmetic, ties everywhere (bisection path)
    (16, 2, 40, 1, "dup"),           # k = 1, duplicated sub-keys (exact ties across blocks)
    (10, 1, 100, 32, "right_zero"),  # all right halves tie: ties of whole rows of keys
    (9, 1, 1024, 32, "normal"),      # 1024^2 keys: 4096 blocks
]


@pytest.mark.parametrize("case", FLAT_EDGE, ids=[f"T{c[0]}H{c[1]}n{c[2]}k{c[3]}-{c[4]}" for c in FLAT_EDGE])
def test_flat_edge(orc, case):
    T, H, n, k, kind = case
    inp = pkm_inputs.custom(T, H, n, k, 512, 16, dtype="bf16", seed=T * 31 + n, kind=kind)
    _flat_parity(orc, inp, k)
    if kind == "integer":
        import product_key_memory_amd as pk
        dev = gpu_util.device()
        q, keys, values = (gpu_util.to_dev(inp[x], dev) for x in ("q", "keys", "values"))
        _, idx, _, _ = pk.pkm_flat_forward(q, keys, values, k)
        ref = orc.forward(inp["q"], inp["keys"], inp["values"], k)
        assert np.array_equal(gpu_util.to_host(idx), ref["idx"]), "exact-arithmetic order differs"


def test_flat_shared_codebooks_equal_replicated():
    """PKM_KEYS_SHARED: one codebook pair [2][n][d_k/2] for all heads gives the
    same bits as that pair replicated into every head's slot (the same
    arithmetic on the same numbers; the kernel reads the pair with a head
    stride of 0)."""
    import product_key_memory_amd as pk
    dev = gpu_util.device()
    inp = pkm_inputs.custom(37, 3, 48, 8, 512, 16, dtype="bf16", seed=4711, kind="normal")
    H = inp["w"].H
    shared = np.ascontiguousarray(inp["keys"][0])
    rep = np.ascontiguousarray(np.broadcast_to(shared, (H,) + shared.shape))
    print(f"[flat shared] T=37 H={H} n=48 k=8", flush=True)
    q, values = gpu_util.to_dev(inp["q"], dev), gpu_util.to_dev(inp["values"], dev)
    out_s = pk.pkm_flat_forward(q, gpu_util.to_dev(shared, dev), values, 8)
    out_r = pk.pkm_flat_forward(q, gpu_util.to_dev(rep, dev), values, 8)
    torch.cuda.synchronize()
    for name, a, b in zip(("y", "idx", "weights", "scores"), out_s, out_r):
        assert torch.equal(a, b), f"{name}: shared codebooks differ from the replicated ones"


def test_flat_rejects_unsupported():
    import product_key_memory_amd as pk
    from product_key_memory_amd import PKMError
    dev = gpu_util.device()
    q = torch.zeros((4, 1, 256), dtype=torch.bfloat16, device=dev)
    keys = torch.zeros((1, 2, 64, 128), dtype=torch.bfloat16, device=dev)
    values = torch.zeros((64 * 64, 8), dtype=torch.bfloat16, device=dev)
    with pytest.raises(PKMError):
        pk.pkm_flat_forward(q, keys, values, 4)            # d_k = 256
