#!/usr/bin/env python3
"""Throughput of the product-key memory layer, forward + backward, on one MI355X.

One step = the whole layer forward (selection, gather) and backward (slot sort,
value gradient written in full, softmax backward, query and sub-key gradients)
over one batch of synthetic tokens resident in HBM.  Every stage is
a call into libpkm.so's C ABI on the current stream; HIP events recorded on
that stream between the stages give each kernel's duration inside the timed
region.  Prints ONE JSON line.

    python bench.py [--steps K] [--warmup W] [--workload NAME]
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

import numpy as np

METRIC = "PKM layer tokens/sec fwd+bwd (n=512,H=4,k=32,d=1024); gather HBM GB/s % peak"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense bf16
MFMA_FP32_PEAK_TFLOPS = 157.3
MFMA_FP64_PEAK_TFLOPS = 78.6    # the selection of float32 storage scores on the fp64 MFMA


def parse():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="base-bf16-zipf-bwd")
    ap.add_argument("--cpu-tokens", type=int, default=1024,
                    help="tokens of the same workload the CPU oracle is timed on")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="first run 3 plain elementwise copies of 256 MiB (bitwise not), whose "
                         "FETCH_SIZE/WRITE_SIZE counters calibrate those of the kernels")
    ap.add_argument("--sweep", action="store_true",
                    help="instead of the bench line: the step (forward + backward) over heads "
                         "H in 1, 2, 4, 8 and picks k in 8, 16, 32 on the workload's other shapes, "
                         "one JSON line each with tokens/s and the fraction of slots in use")
    ap.add_argument("--flat", action="store_true",
                    help="instead of the bench line: the selection by product keys against the "
                         "flat search over all n^2 keys (pkm_flat_forward_select) for n in 128, "
                         "256, 512 at the workload's other shapes, --flat-tokens tokens; one JSON "
                         "line per n")
    ap.add_argument("--flat-tokens", type=int, default=4096)
    ap.add_argument("--record-counters", nargs=4, metavar=("PMC_A", "PMC_B", "PMC_DRAM", "TRACE"),
                    help="no GPU work: read the csv output directories of the three rocprofv3 "
                         "--pmc passes (COUNTER_PASSES) and of a --kernel-trace pass of this "
                         "bench, and write the per-kernel counter table to "
                         "profiles/pkm_counters_<workload>.md")
    ap.add_argument("--record-layer", nargs=2, metavar=("TRACE", "BENCH_LOG"),
                    help="no GPU work: from the csv output directory of a rocprofv3 "
                         "--kernel-trace --stats pass of this bench, the recorded traffic and "
                         "the log of a plain run, write profiles/pkm_layer_<workload>.md")
    ap.add_argument("--record-traffic", nargs=2, metavar=("FETCH_DB", "WRITE_DB"),
                    help="no GPU work: read the rocprofv3 databases of a FETCH_SIZE run and a "
                         "WRITE_SIZE run of `bench.py --calibrate-copy`, and write the "
                         "calibrated HBM bytes per stage to " + "profiles/hbm_traffic_<workload>.json")
    return ap.parse_args()


STAGES = ["select", "gather", "slot_sort", "bwd_values", "bwd_queries"]
# kernels of each stage (name prefixes inside namespace pkm)
STAGE_KERNELS = {
    "select": ("fwd_topk_half_kernel", "fwd_merge_kernel", "fwd_select_kernel"),
    "gather": ("fwd_gather_kernel",),
    "slot_sort": ("bucket_hist_kernel", "bucket_colscan_kernel", "bucket_scatter_kernel",
                  "bucket_sort_kernel"),
    "bwd_values": ("seg_value_kernel", "slot_scan_kernel", "long_run_kernel"),
    "bwd_queries": ("bwd_query_kernel", "dkeys_mfma_kernel", "dkeys_reduce_kernel"),
}
# the value side of pkm_backward_sgd (timed after the step; in the traffic
# record only): the seg_value instance whose SGD flag is true, the slot scan
# without the zeroing of untouched rows (mode 1; the step overwrites, mode 0)
# and the long-run sums of mode 2
SGD_VALUE_KERNELS = {"seg_value_kernel": "true>", "slot_scan_kernel": "1>",
                     "long_run_kernel": "2>"}


def stage_of(short: str):
    """The stage a kernel (name without namespace and arguments) belongs to."""
    base = short.split("<")[0]
    if base in SGD_VALUE_KERNELS and short.replace(" ", "").endswith(SGD_VALUE_KERNELS[base]):
        return "bwd_values_sgd"
    for stage, prefixes in STAGE_KERNELS.items():
        if base in prefixes:
            return stage
    return None
PROFILES = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles")


def sig(x: float, digits: int = 4) -> float:
    """x rounded to `digits` significant digits (small rates stay visible)."""
    return float(f"{x:.{digits}g}")


def traffic_file(workload: str) -> str:
    return os.path.join(PROFILES, f"hbm_traffic_{workload}.json")


def stage_bytes(w, elt: int, touched: int) -> dict:
    """Algorithmic work of one launch of each stage (what its formulation must
    move, cache hits not subtracted; `touched` = memory slots picked at least
    once in the batch)."""
    T, H, k, n, d_k, d_v, half = w.T, w.H, w.k, w.n, w.d_k, w.d_v, w.d_k // 2
    picks, slots = T * H * k, n * n
    return {
        "select": {"flops": 2 * T * H * 2 * n * half,
                   "bytes": T * H * d_k * elt + H * 2 * n * half * elt + picks * 12},
        # one value row per pick, y written once, idx + weights read
        "gather": {"bytes": picks * d_v * elt + T * d_v * elt + picks * 8},
        # idx read twice, order written, counts/cursors/starts per slot
        "slot_sort": {"bytes": picks * 12 + slots * 16},
        # each touched value row read once, every dvalues row written once
        # (overwrite mode), one dy row per pick, per-pick metadata
        "bwd_values": {"bytes": touched * d_v * elt + slots * d_v * 4 + picks * d_v * elt
                       + picks * 16 + slots * 4},
        # q once, sub-keys once, per-pick metadata, dq written, (i, g) lists
        # written and read, partial sub-key sums written and read
        "bwd_queries": {"bytes": T * H * d_k * elt + H * 2 * n * half * elt + picks * 12
                        + T * H * d_k * 4 + T * H * 2 * k * 8 * 2 + H * 2 * n * half * 4 * 3},
    }


def source_hash() -> str:
    import glob
    import hashlib
    hsh = hashlib.sha256()
    csrc = os.path.join(os.path.dirname(os.path.abspath(__file__)), "product_key_memory_amd", "csrc")
    for f in sorted(glob.glob(os.path.join(csrc, "*"))):
        with open(f, "rb") as fh:
            hsh.update(os.path.basename(f).encode() + fh.read())
    return hsh.hexdigest()


def measured_traffic(workload: str) -> dict:
    """HBM bytes per stage from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE
    runs, only if they were taken on the kernels as they are now."""
    try:
        with open(traffic_file(workload)) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return {}
    if rec.get("source_sha256") != source_hash() or rec.get("workload") != workload:
        return {}
    return rec.get("stages", {})


def _counter_means(db: str, counter: str) -> dict:
    """Mean value per dispatch of `counter`, by kernel name, from a rocprofv3
    database (its counters_collection view)."""
    import sqlite3
    con = sqlite3.connect(db)
    rows = con.execute("select kernel_name, avg(value), count(*) from counters_collection "
                       "where counter_name = ? group by kernel_name", (counter,)).fetchall()
    con.close()
    return {name: (float(avg), int(cnt)) for name, avg, cnt in rows}


def _calibration_values(db: str, counter: str) -> list:
    """Per-dispatch values of `counter` for the calibration copy (the only
    bitwise-not kernel the bench runs)."""
    import sqlite3
    con = sqlite3.connect(db)
    rows = con.execute("select value from counters_collection where counter_name = ? and "
                       "kernel_name like '%bitwise_not%'", (counter,)).fetchall()
    con.close()
    return sorted(float(v) for (v,) in rows)


def record_traffic(fetch_db: str, write_db: str, workload: str) -> str:
    """FETCH_SIZE and WRITE_SIZE (KiB per dispatch) of every stage's kernels,
    each scaled by the ratio of the known size of the calibration copy
    (bitwise not over 64 Mi int32: 256 MiB read, 256 MiB written) to the
    median of what the same counter read for its dispatches; summed per stage:
    bytes per launch of the stage."""
    fetch, write = _counter_means(fetch_db, "FETCH_SIZE"), _counter_means(write_db, "WRITE_SIZE")
    copy_kib = 256 * 1024

    def calib(db, counter):
        vals = _calibration_values(db, counter)
        if not vals:
            raise SystemExit("no calibration copy in the database (run bench.py --calibrate-copy)")
        return copy_kib / vals[len(vals) // 2]

    f_fac, w_fac = calib(fetch_db, "FETCH_SIZE"), calib(write_db, "WRITE_SIZE")
    stages = {stage: {"read_bytes": 0, "write_bytes": 0, "kernels": {}}
              for stage in list(STAGE_KERNELS) + ["bwd_values_sgd"]}
    for table, fac, key in ((fetch, f_fac, "read_bytes"), (write, w_fac, "write_bytes")):
        for name, (kib, cnt) in table.items():
            short = name.split("(")[0].replace("void ", "").replace("pkm::", "")
            stage = stage_of(short)
            if stage is None:
                continue
            b = int(round(kib * fac * 1024))
            stages[stage][key] += b
            stages[stage]["kernels"].setdefault(short, {})[key] = b
    out = {"source_sha256": source_hash(), "workload": workload,
           "calibration": {"copy_bytes_read": copy_kib * 1024, "copy_bytes_written": copy_kib * 1024,
                           "fetch_factor": round(f_fac, 4), "write_factor": round(w_fac, 4)},
           "units": "bytes per launch of the stage (the sum of its kernels' dispatches)",
           "stages": stages}
    path = traffic_file(workload)
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    return path


# The three counter passes --record-counters reads (each within one pass's
# limits: at most 8 SQ and 4 TCC counters).  Work counters (instructions,
# busy cycles, hits) do not depend on the pass's timing; the durations come
# from a kernel-trace pass of its own, and every rate is taken against the
# nominal peak clock, 2.4 GHz: no clock is derived from the counters.
COUNTER_PASSES = {
    "A": ["SQ_WAVES", "SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_LDS",
          "SQ_INSTS_SALU", "SQ_INSTS_VMEM_RD", "SQ_INSTS_VMEM_WR"],
    "B": ["SQ_LDS_BANK_CONFLICT", "SQ_ACTIVE_INST_LDS", "SQ_WAIT_INST_ANY", "SQ_ACTIVE_INST_ANY",
          "SQ_WAVE_CYCLES", "SQ_BUSY_CYCLES", "TCC_HIT_sum", "TCC_MISS_sum"],
    # L2 requests to the DRAM address space, in 32-byte units
    "DRAM": ["TCC_EA0_RDREQ_DRAM_32B_sum", "TCC_EA0_WRREQ_WRITE_DRAM_32B_sum"],
}
PEAK_CLOCK_HZ = 2.4e9
SIMDS = 1024


def _short_name(name: str) -> str:
    return name.split("(")[0].replace("void ", "").replace("pkm::", "").strip()


def _csv_rows(directory: str, suffix: str) -> list:
    import csv
    import glob
    rows = []
    for f in sorted(glob.glob(os.path.join(directory, "**", "*" + suffix), recursive=True)):
        with open(f, newline="") as fh:
            rows.extend(csv.DictReader(fh))
    return rows


def record_counters(pmc_a: str, pmc_b: str, pmc_dram: str, trace: str, workload: str) -> str:
    """Per kernel: median duration of its dispatches in the trace pass (a
    cold first dispatch does not move it); means of the counters per
    dispatch in the three counter passes; rates against 1024 SIMDs x
    duration x 2.4 GHz."""
    import statistics
    dur, calls = {}, {}
    for r in _csv_rows(trace, "kernel_trace.csv"):
        k = _short_name(r["Kernel_Name"])
        dur.setdefault(k, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9)
    cnt = {}
    for d in (pmc_a, pmc_b, pmc_dram):
        per = {}
        for r in _csv_rows(d, "counter_collection.csv"):
            key = (_short_name(r["Kernel_Name"]), r["Dispatch_Id"])
            per.setdefault(key, {})[r["Counter_Name"]] = float(r["Counter_Value"])
            per[key]["_grid"] = int(r["Grid_Size"])
        for (k, _), vals in per.items():
            acc = cnt.setdefault(k, {})
            for name, v in vals.items():
                acc.setdefault(name, []).append(v)
    lines = []
    for k in sorted(dur, key=lambda k: -statistics.median(dur[k])):
        t = statistics.median(dur[k])
        c = {name: sum(v) / len(v) for name, v in cnt.get(k, {}).items()}
        if "SQ_WAVES" not in c or t < 5e-6:
            continue
        cap = SIMDS * t * PEAK_CLOCK_HZ
        waves = max(c["SQ_WAVES"], 1.0)
        lds = c.get("SQ_ACTIVE_INST_LDS", 0.0)
        hits, miss = c.get("TCC_HIT_sum", 0.0), c.get("TCC_MISS_sum", 0.0)
        rd = 32 * c.get("TCC_EA0_RDREQ_DRAM_32B_sum", 0.0)
        wr = 32 * c.get("TCC_EA0_WRREQ_WRITE_DRAM_32B_sum", 0.0)
        lines.append("| `%s` | %d | %.1f | %.1f | %.1f | %d | %d | %d | %d | %s | %s | %.3f | %.3f | %.2f |" % (
            k, c.get("_grid", 0), t * 1e6,
            100 * c.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / cap,
            100 * 4 * c.get("SQ_INSTS_VALU", 0.0) / cap,
            round(c.get("SQ_INSTS_VALU", 0.0) / waves), round(c.get("SQ_INSTS_MFMA", 0.0) / waves),
            round(c.get("SQ_INSTS_LDS", 0.0) / waves), round(c.get("SQ_INSTS_SALU", 0.0) / waves),
            "%.2f" % (c.get("SQ_LDS_BANK_CONFLICT", 0.0) / lds) if lds else "-",
            "%.1f" % (100 * hits / (hits + miss)) if hits + miss else "-",
            rd / 1e9, wr / 1e9, (rd + wr) / t / 1e12))
    out = os.path.join(PROFILES, f"pkm_counters_{workload}.md")
    with open(out, "w") as f:
        f.write(COUNTERS_HEADER.format(workload=workload, title=workload_title(workload),
                                       wl_arg=workload_arg(workload),
                                       a=" ".join(COUNTER_PASSES["A"]), b=" ".join(COUNTER_PASSES["B"]),
                                       dram=" ".join(COUNTER_PASSES["DRAM"])))
        f.write("\n".join(lines) + "\n")
    return out


def record_layer(trace: str, bench_log: str, workload: str, steps: int, warmup: int) -> str:
    """Kernel table of the trace pass (kernel_stats.csv), the traffic per
    stage from the recorded FETCH_SIZE / WRITE_SIZE runs, and the JSON line
    of a plain run."""
    stats = _csv_rows(trace, "kernel_stats.csv")
    total = sum(float(r["TotalDurationNs"]) for r in stats) or 1.0
    rows = []
    for r in sorted(stats, key=lambda r: -float(r["TotalDurationNs"])):
        share = 100 * float(r["TotalDurationNs"]) / total
        if share < 0.05:
            continue
        rows.append("| `%s` | %s | %.1f | %.1f |" % (_short_name(r["Name"]), r["Calls"],
                                                     float(r["AverageNs"]) / 1e3, share))
    try:
        with open(traffic_file(workload)) as f:
            traffic = json.load(f)
    except (OSError, ValueError):
        traffic = None
    tlines = []
    if traffic:
        cal = traffic["calibration"]
        tlines.append("Calibration: a plain elementwise kernel (bitwise not over 64 Mi int32: 256 MiB "
                      "read, 256 MiB written) in the same runs, the median of its dispatches; factors "
                      "FETCH_SIZE x%.4f, WRITE_SIZE x%.4f.  FETCH_SIZE and WRITE_SIZE count what "
                      "the L2 moves to and from the fabric, that is the MALL (Infinity Cache) or "
                      "HBM: gfx950 has no counter past the MALL, so these are L2<->fabric bytes, "
                      "an upper bound on HBM traffic.\n" % (cal["fetch_factor"], cal["write_factor"]))
        tlines.append("| stage | read GB | written GB | kernels (read / written GB) |")
        tlines.append("|---|---|---|---|")
        for stage, v in traffic["stages"].items():
            ks = ", ".join("`%s` %.3f / %.3f" % (k, kv.get("read_bytes", 0) / 1e9,
                                                 kv.get("write_bytes", 0) / 1e9)
                           for k, kv in sorted(v["kernels"].items()))
            tlines.append("| %s | %.3f | %.3f | %s |" % (stage, v["read_bytes"] / 1e9,
                                                      v["write_bytes"] / 1e9, ks))
        tlines.append("\nSource hash of the kernels these counters belong to: `%s` (bench.py "
                      "reports `traffic` only while the sources still hash to it)." %
                      traffic["source_sha256"])
    line = ""
    with open(bench_log) as f:
        for ln in f:
            if ln.startswith("{") and '"metric"' in ln:
                line = ln.strip()
    out = os.path.join(PROFILES, f"pkm_layer_{workload}.md")
    with open(out, "w") as f:
        f.write(LAYER_HEADER.format(workload=workload, title=workload_title(workload), steps=steps,
                                    warmup=warmup, runs=steps + warmup, wl_arg=workload_arg(workload)))
        f.write("\n".join(rows) + "\n\n## Traffic per stage launch (FETCH_SIZE, WRITE_SIZE; "
                "KiB per dispatch x calibration)\n\n")
        f.write("\n".join(tlines) if tlines else "not recorded for these sources")
        f.write("\n\n## bench.py line (default 20 timed steps, 5 warm-up)\n\n```json\n%s\n```\n" % line)
    return out


def workload_title(workload: str) -> str:
    import pkm_inputs
    w = pkm_inputs.WORKLOADS[workload]
    return f"T={w.T}, H={w.H}, n={w.n}, k={w.k}, d_k={w.d_k}, d_v={w.d_v}, {w.dtype}"


LAYER_HEADER = """# PKM layer, fwd+bwd, `{workload}` ({title}): kernel trace and traffic

One MI355X (gfx950), one process.  Inputs seeded and synthetic
(`pkm_inputs.py`), resident in HBM.  Step = forward (selection, gather) +
backward (slot sort, value side with dvalues overwritten, query side).

## Commands (from the repository root; `<out>` is any output directory)

```
python3 bench.py{wl_arg} > <out>/bench.log
rocprofv3 --kernel-trace --stats -d <out>/lay_t -o t --output-format csv -- python3 bench.py{wl_arg} --steps {steps} --warmup {warmup} --no-cpu-baseline
rocprofv3 --pmc FETCH_SIZE -d <out>/prof_fetch -o fetch -- python3 bench.py{wl_arg} --steps 2 --warmup 1 --no-cpu-baseline --calibrate-copy
rocprofv3 --pmc WRITE_SIZE -d <out>/prof_write -o write -- python3 bench.py{wl_arg} --steps 2 --warmup 1 --no-cpu-baseline --calibrate-copy
python3 bench.py{wl_arg} --record-traffic <out>/prof_fetch/fetch_results.db <out>/prof_write/write_results.db
python3 bench.py{wl_arg} --record-layer <out>/lay_t <out>/bench.log
```

## Kernel trace (kernel_stats of the trace pass; the step's kernels run {runs} times = {warmup} warm-up + {steps} timed steps; after the step the bench times the update, usage, fused-SGD, sweep-free extras and the query network, {runs} runs each)

| kernel | calls | avg µs | share % |
|---|---|---|---|
"""


def workload_arg(workload: str) -> str:
    return "" if workload == "base-bf16-zipf-bwd" else f" --workload {workload}"


COUNTERS_HEADER = """# Per-kernel counters, `{workload}` ({title})

One MI355X (gfx950), one process.  Durations: the median over a kernel's
dispatches in a kernel-trace pass of 2 warm-up and 5 timed steps.  Counters: means per dispatch over three
counter passes (each runs the benchmark for 1 warm-up and 1 timed step; the
kernels and their work are those of the timed runs).  Rates are against the
machine's capacity over the kernel's duration at the nominal 2.4 GHz peak
clock -- no clock is derived from the counters:

* MFMA busy % = `SQ_VALU_MFMA_BUSY_CYCLES` / (1024 SIMDs x duration x 2.4 GHz)
  (16 busy cycles per `v_mfma_f32_16x16x32_bf16`);
* VALU issue % = 4 x `SQ_INSTS_VALU` / (1024 x duration x 2.4 GHz) (a wave64
  VALU instruction holds a 16-lane SIMD for 4 cycles);
* per-wave instruction counts = counter / `SQ_WAVES`; LDS conflict cycles per
  LDS instruction = `SQ_LDS_BANK_CONFLICT` / `SQ_ACTIVE_INST_LDS`; L2 hit =
  `TCC_HIT` / (`TCC_HIT` + `TCC_MISS`);
* DRAM-destined GB = 32 x `TCC_EA0_RDREQ_DRAM_32B` (reads) and 32 x
  `TCC_EA0_WRREQ_WRITE_DRAM_32B` (writes): the L2's requests sorted by
  destination (DRAM, as against GMI or IO).  The MALL (Infinity Cache) sits on
  the memory side of the fabric, so its hits count here as well: gfx950 shows
  no counter past it, and these bytes and their rate (the last column, over
  the kernel's duration) are L2<->fabric figures, an upper bound on what HBM
  itself moved.

Kernels under 5 µs are left out.

## Commands (from the repository root; `<out>` is any output directory)

```
rocprofv3 --kernel-trace --stats -d <out>/cnt_t -o t --output-format csv -- python3 bench.py{wl_arg} --steps 5 --warmup 2 --no-cpu-baseline
rocprofv3 --pmc {a} -d <out>/cnt_a -o p --output-format csv -- python3 bench.py{wl_arg} --steps 1 --warmup 1 --no-cpu-baseline
rocprofv3 --pmc {b} -d <out>/cnt_b -o p --output-format csv -- python3 bench.py{wl_arg} --steps 1 --warmup 1 --no-cpu-baseline
rocprofv3 --pmc {dram} -d <out>/cnt_d -o p --output-format csv -- python3 bench.py{wl_arg} --steps 1 --warmup 1 --no-cpu-baseline
python3 bench.py{wl_arg} --record-counters <out>/cnt_a <out>/cnt_b <out>/cnt_d <out>/cnt_t
```

| kernel | grid | µs | MFMA busy % | VALU issue % | VALU / wave | MFMA / wave | LDS / wave | SALU / wave | LDS conflict cycles / LDS instr | L2 hit % | DRAM-destined read GB | DRAM-destined write GB | L2<->fabric TB/s |
|---|---|---|---|---|---|---|---|---|---|---|---|---|---|
"""


def measure_extras(torch, _lib, p, values, dvalues, slot_start, w, elt, touched, stream) -> dict:
    """The value-table update and the usage counter that follow the backward
    (not part of the step): event time per call over 5 calls after 2 warm-up
    calls, on the step's own gradient and slot sort."""
    slots, d_v = w.n * w.n, w.d_v
    dev = values.device
    m = torch.zeros((slots, d_v), dtype=torch.float32, device=dev)
    v = torch.zeros_like(m)
    counts = torch.zeros(slots, dtype=torch.int64, device=dev)
    used = torch.zeros(1, dtype=torch.int64, device=dev)
    sp = stream.cuda_stream
    P = lambda t: t.data_ptr()  # noqa: E731
    calls = {
        "sparse_sgd": (lambda i: _lib.sparse_sgd(p, P(values), P(dvalues), P(slot_start), 1e-3, sp),
                       touched * d_v * (2 * elt + 4) + (slots + 1) * 4),
        "sparse_adam": (lambda i: _lib.sparse_adam(p, P(values), P(dvalues), P(slot_start), P(m),
                                                   P(v), i + 1, 1e-3, 0.9, 0.999, 1e-8, sp),
                        touched * d_v * (2 * elt + 4 + 16) + (slots + 1) * 4),
        "slot_usage": (lambda i: _lib.slot_usage(p, P(slot_start), P(counts), P(used), sp),
                       (slots + 1) * 4 + slots * 16),
    }
    out = {}
    for name, (fn, nbytes) in calls.items():
        for i in range(2):
            assert fn(i) == 0, name
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(5):
            fn(2 + i)
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / 5
        gbs = nbytes / (ms * 1e-3) / 1e9
        out[name] = {"ms": round(ms, 5), "bytes": nbytes, "GB/s": round(gbs, 1),
                     "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}
    out["slot_usage"]["used_fraction"] = round(int(used.item()) / slots, 4)
    return out


def measure_fused_sgd(torch, _lib, p, bufs, ws, ws_bytes, stream) -> dict:
    """The training backward with its value update: pkm_backward (dvalues
    overwritten) then pkm_sparse_sgd, against pkm_backward_sgd (the update
    fused into the value side, no dvalues array); event time per call over 5
    calls after 2 warm-up calls, on the step's inputs (the values drift by
    lr = 1e-3 per call, the selection is the step's)."""
    q, keys, values, idx, wts, dy, dq, dkeys, dvalues = bufs
    sp = stream.cuda_stream
    P = lambda t: t.data_ptr()  # noqa: E731
    fws_bytes = _lib.workspace_bytes(p, 2)
    fws = torch.empty(max(fws_bytes, 1), dtype=torch.uint8, device=values.device)

    # the update reads the backward's own slot sort: slot_start follows the
    # T*H*k floats of dw in its workspace, rounded up to 256 bytes
    starts = P(ws) + ((p.T * p.H * p.k * 4 + 255) // 256) * 256

    def chain():
        rc = _lib.backward_overwrite(p, P(q), P(keys), P(values), P(idx), P(wts), P(dy), P(dq),
                                     P(dkeys), P(dvalues), P(ws), ws_bytes, sp)
        return rc | _lib.sparse_sgd(p, P(values), P(dvalues), starts, 1e-3, sp)

    def fused():
        return _lib.backward_sgd(p, P(q), P(keys), P(values), P(idx), P(wts), P(dy), P(dq),
                                 P(dkeys), 1e-3, P(fws), fws_bytes, sp)

    out = {}
    for name, fn in (("backward_then_sgd", chain), ("backward_sgd_fused", fused)):
        for _ in range(2):
            assert fn() == 0, name
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(5):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        out[name] = {"ms": round(e0.elapsed_time(e1) / 5, 5)}
    return out


def measure_query_net(torch, _lib, w, dq, stream, d_model: int = 1600) -> dict:
    """The query network q = BN(x W^T) in front of the layer (not part of the
    step, whose q is given): x [T][1600] (the pages' model width) and
    W [H d_k][1600] in the workload's dtype, seeded normal; forward and
    backward (dq of the step) timed with events over 5 calls after 2."""
    dev = dq.device
    D = w.H * w.d_k
    gen = torch.Generator(device=dev).manual_seed(1600)
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    x = torch.randn((w.T, d_model), device=dev, generator=gen).to(tdt)
    W = (torch.randn((D, d_model), device=dev, generator=gen) * d_model ** -0.5).to(tdt)
    qp = _lib.QueryProblem(w.T, d_model, D, 1 if w.dtype == "bf16" else 0, 0)
    nf, nb = _lib.query_workspace_bytes(qp, False), _lib.query_workspace_bytes(qp, True)
    ws = torch.empty(max(nf, nb), dtype=torch.uint8, device=dev)
    q = torch.empty((w.T, D), dtype=tdt, device=dev)
    z = torch.empty((w.T, D), dtype=torch.float32, device=dev)
    mean = torch.empty(D, dtype=torch.float32, device=dev)
    rstd = torch.empty_like(mean)
    dx = torch.empty((w.T, d_model), dtype=torch.float32, device=dev)
    dW = torch.empty((D, d_model), dtype=torch.float32, device=dev)
    dg, db = torch.empty_like(mean), torch.empty_like(mean)
    dq2 = dq.reshape(w.T, D)
    sp = stream.cuda_stream
    P = lambda t: t.data_ptr()  # noqa: E731
    fwd = lambda: _lib.query_forward(qp, P(x), P(W), None, None, 1e-5, P(q), P(z), P(mean),  # noqa: E731
                                     P(rstd), P(ws), nf, sp)
    bwd = lambda: _lib.query_backward(qp, P(x), P(W), None, P(z), P(mean), P(rstd), P(dq2),  # noqa: E731
                                      P(dx), P(dW), P(dg), P(db), P(ws), nb, sp)
    flops = 2 * w.T * d_model * D
    peak = MFMA_BF16_PEAK_TFLOPS if w.dtype == "bf16" else MFMA_FP32_PEAK_TFLOPS
    out = {"d_model": d_model, "d_out": D}
    for name, fn, fl in (("forward", fwd, flops), ("backward", bwd, 2 * flops)):
        for _ in range(2):
            assert fn() == 0, name
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(5):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / 5
        tf = fl / (ms * 1e-3) / 1e12
        out[name] = {"ms": round(ms, 5), "flops": fl, "TFLOP/s": round(tf, 1),
                     "mfma_frac": round(tf / peak, 4)}
        if name == "backward" and w.dtype == "bf16":
            # dz enters both products as two bf16 planes (hi + lo): the MFMAs
            # execute twice the nominal flops
            out[name]["mfma_flops"] = 2 * fl
            out[name]["mfma_work_frac"] = round(2 * tf / peak, 4)
    return out


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def cpu_baseline(inp, k: int, count: int) -> dict:
    import oracle
    import pkm_inputs
    orc = oracle.default()
    w = inp["w"]
    sub = pkm_inputs.token_subset(w.T, count, seed=4242)
    q = inp["q"][sub]
    dy = inp["dy"][sub]
    t0 = time.perf_counter()
    ref = orc.forward(q, inp["keys"], inp["values"], k)
    orc.backward(q, inp["keys"], inp["values"], ref["idx"], ref["weights"], dy)
    dt = time.perf_counter() - t0
    return {"value": len(sub) / dt, "unit": "tokens/s", "cores": orc.max_threads(),
            "kind": "oracle",
            "sample": f"{len(sub)} seeded tokens of {w.name}, forward+backward in float64: flat "
                      f"scoring and full sort of all {w.n * w.n} slots per head, dense gradients; "
                      f"{dt:.2f} s wall on {orc.max_threads()} threads ({_cpu_model()})"}


def run_sweep(args) -> None:
    """The speed / memory-use knobs: heads H and picks k on the workload's
    remaining shapes (synthetic inputs of the same recipe, one draw per H),
    and at k = 32 one codebook pair shared by the heads (the first head's).
    Per point: W warm-up and K timed steps of pkm_forward + pkm_backward_overwrite
    (dvalues overwritten) bracketed by events, and the share of the n*n slots
    some pick selected in the batch."""
    import dataclasses

    import torch
    import pkm_inputs
    from product_key_memory_amd import _lib
    from product_key_memory_amd.pkm import problem

    dev = torch.device("cuda", 0)
    base = pkm_inputs.WORKLOADS[args.workload]
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream
    P = lambda t: t.data_ptr()  # noqa: E731
    for H in (1, 2, 4, 8):
        w0 = dataclasses.replace(base, H=H, name=f"{base.name}-H{H}")
        inp = pkm_inputs.make(w0, with_dy=True)
        tdt = torch.bfloat16 if w0.dtype == "bf16" else torch.float32

        def to_dev(a):
            t = torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).to(dev)
            return t.view(torch.bfloat16) if a.dtype == np.uint16 else t

        q, keys, values, dy = (to_dev(inp[x]) for x in ("q", "keys", "values", "dy"))
        del inp
        T, n, d_k, d_v = w0.T, w0.n, w0.d_k, w0.d_v
        y = torch.empty((T, d_v), dtype=tdt, device=dev)
        dvalues = torch.empty((n * n, d_v), dtype=torch.float32, device=dev)
        dq = torch.empty((T, H, d_k), dtype=torch.float32, device=dev)
        dkeys = torch.empty((H, 2, n, d_k // 2), dtype=torch.float32, device=dev)
        keys_one = keys[0].contiguous()          # one codebook pair for every head
        for k, shared in ((8, False), (16, False), (32, False), (32, True)):
            p = problem(T, H, n, k, d_k, d_v, tdt, keys_shared=shared)
            kp = P(keys_one) if shared else P(keys)
            fb, bb = _lib.workspace_bytes(p, False), _lib.workspace_bytes(p, True)
            fws = torch.empty(max(fb, 1), dtype=torch.uint8, device=dev)
            bws = torch.empty(max(bb, 1), dtype=torch.uint8, device=dev)
            idx = torch.empty((T, H, k), dtype=torch.int32, device=dev)
            wts = torch.empty((T, H, k), dtype=torch.float32, device=dev)

            def step():
                rc = _lib.forward(p, P(q), kp, P(values), P(y), P(idx), P(wts), None,
                                  P(fws), fb, sp)
                rc |= _lib.backward_overwrite(p, P(q), kp, P(values), P(idx), P(wts), P(dy),
                                              P(dq), P(dkeys), P(dvalues), P(bws), bb, sp)
                if rc:
                    raise RuntimeError(f"libpkm returned {rc}")

            for _ in range(args.warmup):
                step()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(args.steps):
                step()
            e1.record(stream)
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / args.steps
            used = torch.unique(idx).numel() / (n * n)
            print(json.dumps({"sweep": {"workload": base.name, "H": H, "k": k,
                                        "codebooks": "shared" if shared else "per head"},
                              "tokens_per_s": round(T / (ms * 1e-3), 1),
                              "ms_per_step": round(ms, 4), "used_fraction": round(used, 4)}),
                  flush=True)
        del q, keys, values, dy, y, dvalues, dq, dkeys
        torch.cuda.empty_cache()


def run_flat(args) -> None:
    """Search cost, flat against product keys (companion page, "Search cost:
    flat vs product keys"): the workload's recipe at --flat-tokens tokens and
    n = 128, 256, 512; per n, W warm-up and K timed calls of the product-key selection and 1 warm-up
    and max(2, K / 4) timed calls of the flat search
    (scores, top-k, softmax; the gather that follows is the same for both)
    bracketed by events.  Flops: product keys 2 T H 2 n (d_k / 2), flat
    2 T H n^2 d_k.  The sets of the two searches are compared (equal wherever
    the k-th / (k+1)-th gap is clear; the parity tests check that)."""
    import dataclasses

    import torch
    import pkm_inputs
    from product_key_memory_amd import _lib
    from product_key_memory_amd.pkm import problem

    dev = torch.device("cuda", 0)
    base = pkm_inputs.WORKLOADS[args.workload]
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream
    P = lambda t: t.data_ptr()  # noqa: E731
    for n in (128, 256, 512):
        w0 = dataclasses.replace(base, n=n, T=args.flat_tokens, zipf=0.0, backward=False,
                                 name=f"{base.name}-n{n}-T{args.flat_tokens}")
        inp = pkm_inputs.make(w0, with_dy=False)
        q = torch.from_numpy(inp["q"].view(np.int16)).to(dev).view(torch.bfloat16)
        keys = torch.from_numpy(inp["keys"].view(np.int16)).to(dev).view(torch.bfloat16)
        T, H, k, d_k = w0.T, w0.H, w0.k, w0.d_k
        p = problem(T, H, n, k, d_k, w0.d_v, torch.bfloat16)
        fb = _lib.workspace_bytes(p, False)
        fws = torch.empty(max(fb, 1), dtype=torch.uint8, device=dev)
        out = {name: (torch.empty((T, H, k), dtype=torch.int32, device=dev),
                      torch.empty((T, H, k), dtype=torch.float32, device=dev))
               for name in ("product", "flat")}
        calls = {
            "product": lambda: _lib.forward_select(p, P(q), P(keys), P(out["product"][0]),
                                                   P(out["product"][1]), None, P(fws), fb, sp),
            "flat": lambda: _lib.flat_forward_select(p, P(q), P(keys), P(out["flat"][0]),
                                                     P(out["flat"][1]), None, sp),
        }
        flops = {"product": 2 * T * H * 2 * n * (d_k // 2), "flat": 2 * T * H * n * n * d_k}
        res = {}
        for name, fn in calls.items():
            steps = args.steps if name == "product" else max(2, args.steps // 4)
            for _ in range(args.warmup if name == "product" else 1):
                assert fn() == 0, name
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(steps):
                fn()
            e1.record(stream)
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / steps
            tf = flops[name] / (ms * 1e-3) / 1e12
            res[name] = {"ms": round(ms, 4), "tokens_per_s": round(T / (ms * 1e-3), 1),
                         "flops": flops[name], "TFLOP/s": round(tf, 1),
                         "mfma_frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4)}
        same = (out["product"][0].sort(dim=2).values == out["flat"][0].sort(dim=2).values)
        same_rows = float(same.all(dim=2).float().mean().item())
        print(json.dumps({"flat_vs_product": {"workload": w0.name, "T": T, "H": H, "n": n,
                                              "keys": n * n, "k": k, "d_k": d_k},
                          "product": res["product"], "flat": res["flat"],
                          "flat_over_product_time": round(res["flat"]["ms"] / res["product"]["ms"], 1),
                          "identical_sets": round(same_rows, 5)}), flush=True)
        del q, keys, fws, out
        torch.cuda.empty_cache()


def main():
    args = parse()
    if args.record_traffic:
        print(record_traffic(*args.record_traffic, args.workload))
        return
    if args.record_layer:
        print(record_layer(*args.record_layer, args.workload, args.steps, args.warmup))
        return
    if args.record_counters:
        print(record_counters(*args.record_counters, args.workload))
        return
    if args.sweep:
        run_sweep(args)
        return
    if args.flat:
        run_flat(args)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(the sharding design is described in the design notes); run with --gpus 1",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import pkm_inputs
    from product_key_memory_amd import _lib
    from product_key_memory_amd.pkm import problem

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda", 0)
    _lib.lib()                                   # fail loudly if libpkm.so is missing

    inp = pkm_inputs.make(args.workload, with_dy=True)
    w = inp["w"]
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    elt = 2 if w.dtype == "bf16" else 4

    def to_dev(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

    q, keys, values, dy = (to_dev(inp[x]) for x in ("q", "keys", "values", "dy"))
    T, H, n, k, d_k, d_v = w.T, w.H, w.n, w.k, w.d_k, w.d_v
    y = torch.empty((T, d_v), dtype=tdt, device=dev)
    idx = torch.empty((T, H, k), dtype=torch.int32, device=dev)
    wts = torch.empty((T, H, k), dtype=torch.float32, device=dev)
    scores = torch.empty((T, H, k), dtype=torch.float32, device=dev)
    dw = torch.empty((T, H, k), dtype=torch.float32, device=dev)
    slot_start = torch.empty(n * n + 1, dtype=torch.int32, device=dev)
    order = torch.empty((T * H * k,), dtype=torch.int32, device=dev)
    dq = torch.empty((T, H, d_k), dtype=torch.float32, device=dev)
    dkeys = torch.empty((H, 2, n, d_k // 2), dtype=torch.float32, device=dev)
    dvalues = torch.empty((n * n, d_v), dtype=torch.float32, device=dev)
    p = problem(T, H, n, k, d_k, d_v, tdt)
    ws_bytes = _lib.workspace_bytes(p, True)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    fws_bytes = _lib.workspace_bytes(p, False)
    fws = torch.empty(max(fws_bytes, 1), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream
    P = lambda t: t.data_ptr()  # noqa: E731

    def step(ev=None):
        def mark(i):
            if ev is not None:
                ev[i].record(stream)
        mark(0)
        rc = _lib.forward_select(p, P(q), P(keys), P(idx), P(wts), P(scores), P(fws), fws_bytes,
                                 sp)
        mark(1)
        rc |= _lib.forward_gather(p, P(values), P(idx), P(wts), P(y), sp)
        mark(2)
        rc |= _lib.slot_sort(p, P(idx), P(slot_start), P(order), P(ws), ws_bytes, sp)
        mark(3)
        rc |= _lib.backward_values(p, P(values), P(idx), P(wts), P(dy), P(slot_start), P(order),
                                   P(dvalues), 0, P(dw), P(ws), ws_bytes, sp)   # overwritten
        mark(4)
        rc |= _lib.backward_queries(p, P(q), P(keys), P(idx), P(wts), P(dw), P(dq), P(dkeys),
                                    P(ws), ws_bytes, sp)
        mark(5)
        if rc:
            raise RuntimeError(f"libpkm returned {rc}")

    if args.calibrate_copy:
        # a plain elementwise kernel of known size (reads 256 MiB, writes 256 MiB,
        # 16-byte accesses like the layer's own kernels), of a kind the bench
        # runs nowhere else, so its dispatches are easy to find
        src = torch.ones(64 << 20, dtype=torch.int32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.bitwise_not(src, out=dst)
        torch.cuda.synchronize()
        del src, dst

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    nev = len(STAGES) + 1
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(nev)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(events[s])
    torch.cuda.synchronize()
    t1 = time.perf_counter()

    per_stage = {name: 0.0 for name in STAGES}
    for ev in events:
        for i, name in enumerate(STAGES):
            per_stage[name] += ev[i].elapsed_time(ev[i + 1])
    per_stage = {name: v / args.steps for name, v in per_stage.items()}   # ms per launch
    wall_ms = (t1 - t0) * 1e3 / args.steps
    tokens_per_s = T / (wall_ms * 1e-3)

    touched = int(((slot_start[1:] - slot_start[:-1]) > 0).sum().item())
    work = stage_bytes(w, elt, touched)
    traffic = measured_traffic(w.name)
    kernels = {}
    for name in STAGES:
        ms = per_stage[name]
        gbs = work[name]["bytes"] / (ms * 1e-3) / 1e9
        entry = {"ms": round(ms, 5), "bytes": work[name]["bytes"], "GB/s": sig(gbs),
                 "hbm_frac": sig(gbs / HBM_PEAK_GBS)}
        if "flops" in work[name]:
            # the contraction's own peak: bf16 MFMA, or (float32 storage) the
            # fp64 MFMA the selection scores with
            tf = work[name]["flops"] / (ms * 1e-3) / 1e12
            peak = MFMA_BF16_PEAK_TFLOPS if w.dtype == "bf16" else MFMA_FP64_PEAK_TFLOPS
            entry.update({"flops": work[name]["flops"], "TFLOP/s": sig(tf),
                          "mfma_peak": peak, "mfma_frac": sig(tf / peak)})
        if name in traffic:
            entry["traffic"] = traffic[name]["read_bytes"] + traffic[name]["write_bytes"]
        kernels[name] = entry

    extras = measure_extras(torch, _lib, p, values, dvalues, slot_start, w, elt, touched, stream)
    extras.update(measure_fused_sgd(torch, _lib, p, (q, keys, values, idx, wts, dy, dq, dkeys,
                                                     dvalues), ws, ws_bytes, stream))
    query_net = measure_query_net(torch, _lib, w, dq, stream)

    dominant = max(STAGES, key=lambda s: per_stage[s])
    dk = kernels[dominant]
    if "flops" in dk:
        # a contraction (the selection's scoring) is priced against its MFMA peak
        roofline = {"kernel": dominant, "bound": "mfma", "achieved": dk["TFLOP/s"],
                    "peak": dk["mfma_peak"], "unit": "TFLOP/s", "frac": dk["mfma_frac"],
                    "traffic": dk.get("traffic")}
    else:
        roofline = {"kernel": dominant, "bound": "hbm", "achieved": dk["GB/s"],
                    "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": dk["hbm_frac"], "traffic": dk.get("traffic")}

    out = {
        "metric": METRIC,
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "tokens": T, "heads": H, "n": n, "slots": n * n, "k": k,
                   "d_k": d_k, "d_v": d_v, "storage": w.dtype, "accumulate": "fp32",
                   "zipf": w.zipf, "touched_slots": touched,
                   "step": "forward + backward (dvalues overwritten)"},
        "gather": {"GB/s": kernels["gather"]["GB/s"], "hbm_frac": kernels["gather"]["hbm_frac"]},
        # the forward alone (selection + gather, from the same stage events)
        "forward_tokens_per_s": round(T / ((kernels["select"]["ms"] + kernels["gather"]["ms"]) * 1e-3), 1),
        "roofline": roofline,
        "kernels": kernels,
        "after_backward": extras,
        "query_network": query_net,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(inp, k, args.cpu_tokens)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
