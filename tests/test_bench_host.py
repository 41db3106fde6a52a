"""Host logic of bench.py, on the CPU: the one-GPU refusal, the algorithmic
work per stage that `roofline.achieved` is built on (the figures the design
notes quote for T = 16384, H = 4, n = 512, k = 32, d_k = 512, d_v = 1024,
bf16), the rounding of rates, and the rule that recorded traffic counts are
used only for the kernel sources they were taken on."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import pkm_inputs  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_stage_work_of_the_base_workload():
    w = pkm_inputs.WORKLOADS["base-bf16-zipf-bwd"]
    work = bench.stage_bytes(w, 2, touched=259176)
    # 2 T H 2 n (d_k / 2) multiply-adds counted as two flops each
    assert work["select"]["flops"] == 34_359_738_368
    # 2,097,152 value rows of 2 KiB, y once, idx and weights once
    assert work["gather"]["bytes"] == 4_345_298_944
    # touched rows once, 1 GiB of float32 dvalues, one dy row per pick, metadata
    assert work["bwd_values"]["bytes"] == 5_934_104_576


def test_rates_keep_four_significant_digits():
    assert bench.sig(0.0036412) == 0.003641
    assert bench.sig(6979.04) == 6979.0
    assert bench.sig(0.109523) == 0.1095
    assert bench.sig(0.0) == 0.0


def test_traffic_only_for_the_sources_it_was_taken_on(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    stages = {"gather": {"read_bytes": 1, "write_bytes": 2}}
    rec = {"workload": "wl", "source_sha256": bench.source_hash(), "stages": stages}
    (tmp_path / "hbm_traffic_wl.json").write_text(json.dumps(rec))
    assert bench.measured_traffic("wl") == stages
    rec["source_sha256"] = "0" * 64
    (tmp_path / "hbm_traffic_wl.json").write_text(json.dumps(rec))
    assert bench.measured_traffic("wl") == {}
    assert bench.measured_traffic("missing") == {}


@pytest.mark.parametrize("name", ["base-bf16-zipf-bwd", "proj-fp32", "tiny-fp32"])
def test_committed_traffic_record_names_its_workload(name):
    with open(bench.traffic_file(name)) as f:
        rec = json.load(f)
    assert rec["workload"] == name
    assert len(rec["source_sha256"]) == 64
