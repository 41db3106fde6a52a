"""The backward gives the same bits on every run (no float atomics; the picks
of a slot meet in ascending pick id; the pieces of a hot slot's long run are
added in a fixed order), at the benchmark workload: 16384 tokens, 4 heads,
512^2 slots, k = 32, d_v = 1024, bf16, Zipf-biased queries (slots picked
thousands of times, far more than one wave's share)."""
import pytest
import torch

import gpu_util
import pkm_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def bench_inputs():
    dev = gpu_util.device()
    inp = pkm_inputs.make("base-bf16-zipf-bwd")
    w = inp["w"]
    print(f"[determinism] {w.name}", flush=True)
    t = {x: gpu_util.to_dev(inp[x], dev) for x in ("q", "keys", "values", "dy")}
    import product_key_memory_amd as pk
    _, idx, wts, _ = pk.pkm_forward(t["q"], t["keys"], t["values"], w.k)
    t.update(idx=idx, wts=wts, w=w)
    return t


def test_backward_overwrite_and_accumulate_repeat_bitwise(bench_inputs):
    import product_key_memory_amd as pk
    t = bench_inputs
    args = (t["q"], t["keys"], t["values"], t["idx"], t["wts"], t["dy"])
    runs = [pk.pkm_backward(*args) for _ in range(2)]          # overwrite mode
    start = torch.randn_like(runs[0][2])
    acc = [start.clone(), start.clone()]
    for a in acc:                                               # accumulate mode
        pk.pkm_backward(*args, dvalues=a)
    torch.cuda.synchronize()
    for name, x, y in zip(("dq", "dkeys", "dvalues"), runs[0], runs[1]):
        assert torch.equal(x, y), f"{name} differs between two runs"
    assert torch.equal(acc[0], acc[1]), "accumulated dvalues differ between two runs"
    # the hottest slot is picked far more often than one wave's share of 256
    counts = torch.bincount(t["idx"].reshape(-1).long(), minlength=t["w"].slots)
    assert int(counts.max()) > 4 * 256


def test_backward_sgd_repeats_bitwise(bench_inputs):
    import product_key_memory_amd as pk
    t = bench_inputs
    outs = []
    for _ in range(2):
        vals = t["values"].clone()
        dq, dkeys = pk.pkm_backward_sgd(t["q"], t["keys"], vals, t["idx"], t["wts"], t["dy"], 1e-2)
        outs.append((vals, dq, dkeys))
    torch.cuda.synchronize()
    for name, x, y in zip(("values", "dq", "dkeys"), outs[0], outs[1]):
        assert torch.equal(x, y), f"{name} differs between two runs of pkm_backward_sgd"
    assert not torch.equal(outs[0][0], t["values"]), "the update changed nothing"
