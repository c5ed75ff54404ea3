"""bench.py --summarize-counters on synthetic rocprofv3 output (no GPU): every
bench workload's summary step runs to completion on CSV files laid out and
headed as rocprofv3 writes them, and its derived figures follow from the
numbers planted in them (clock from GRBM_GUI_ACTIVE, MFMA busy, copy-calibrated
HBM bytes).  This catches host-side errors of the counter pipeline before a
GPU lease is spent on it."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

KT_HEAD = ["Kind", "Agent_Id", "Queue_Id", "Stream_Id", "Thread_Id", "Dispatch_Id", "Kernel_Id", "Kernel_Name",
           "Correlation_Id", "Start_Timestamp", "End_Timestamp", "LDS_Block_Size", "Scratch_Size", "VGPR_Count",
           "Accum_VGPR_Count", "SGPR_Count", "Workgroup_Size_X", "Workgroup_Size_Y", "Workgroup_Size_Z",
           "Grid_Size_X", "Grid_Size_Y", "Grid_Size_Z"]
ST_HEAD = ["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs", "MaxNs", "StdDev"]
CC_HEAD = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id", "Grid_Size",
           "Kernel_Id", "Kernel_Name", "Workgroup_Size", "LDS_Block_Size", "Scratch_Size", "VGPR_Count",
           "Accum_VGPR_Count", "SGPR_Count", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]

DUR_NS = 1_000_000          # every planted dispatch lasts 1 ms
CLOCK_GHZ = 2.0             # GRBM_GUI_ACTIVE planted for this clock
MFMA_BUSY = 0.5
COPY_MIB = bench.COPY_MIB


def _write(path, head, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as fh:
        w = csv.writer(fh, quoting=csv.QUOTE_NONNUMERIC)
        w.writerow(head)
        w.writerows(rows)


def _trace_rows(names, n):
    rows, t, did = [], 1_000_000_000, 1
    for _ in range(n):
        for k in names:
            rows.append(["KERNEL_DISPATCH", "Agent 1", 1, 0, 1, did, 1, k, did, t, t + DUR_NS, 0, 0, 128, 0, 32,
                         256, 1, 1, 1024, 1, 1])
            t += DUR_NS + 1000
            did += 1
    return rows


def _counter_rows(names, n, counters):
    rows, t, did = [], 1_000_000_000, 1
    for _ in range(n):
        for k in names:
            for c, v in counters(k).items():
                rows.append([did, did, "Agent 1", 1, 1, 1, 262144, 1, k, 256, 0, 0, 128, 0, 32, c, float(v), t,
                             t + DUR_NS])
            t += DUR_NS + 1000
            did += 1
    return rows


def _plant(base, wl):
    """Synthetic raw output of collect_counters for workload `wl` under `base`."""
    spec = bench._workload_spec(wl)
    raw = f"{spec['prefix']}_{spec['tag']}"
    # kernel names as the trace would show them (they contain the spec's substrings)
    names = [f"_ZN12_GLOBAL__N_1{len(k)}{k}IDF16bLi128ELb0EEEvNS_6ParamsE" for k in spec["kernels"]]
    steps, psteps = 4, 3
    cycles = CLOCK_GHZ * DUR_NS                       # per XCD during one dispatch
    simd_cycles = bench.CUS * bench.SIMDS_PER_CU * cycles

    def sq(_k):
        out = {c: 1000.0 for p in bench.SQ_PASSES for c in p}
        out.update(GRBM_GUI_ACTIVE=cycles * bench.XCDS, SQ_WAVES=8192.0,
                   SQ_VALU_MFMA_BUSY_CYCLES=MFMA_BUSY * simd_cycles, SQ_VALU_MFMA_COEXEC_CYCLES=0.25 * simd_cycles,
                   SQ_LDS_IDX_ACTIVE=0.3 * bench.CUS * cycles, SQ_LDS_BANK_CONFLICT=0.0)
        return out

    _write(os.path.join(base, f"kt_{raw}", "fa_kernel_trace.csv"), KT_HEAD, _trace_rows(names, steps))
    _write(os.path.join(base, f"kt_{raw}", "fa_kernel_stats.csv"), ST_HEAD,
           [[k, steps, steps * DUR_NS, float(DUR_NS), 100.0 / len(names), DUR_NS, DUR_NS, 0.0] for k in names])
    for i, counters in enumerate(bench.SQ_PASSES):
        d = os.path.join(base, f"sq{i}_{raw}")
        _write(os.path.join(d, "fa_counter_collection.csv"), CC_HEAD,
               _counter_rows(names, psteps, lambda k, c=counters: {n: sq(k)[n] for n in c}))
        if "GRBM_GUI_ACTIVE" in counters:
            _write(os.path.join(d, "fa_kernel_trace.csv"), KT_HEAD, _trace_rows(names, psteps))
    # traffic: each kernel reads 2 MiB and writes 1 MiB in counter units of 2 KiB per count
    for cn, mib in (("FETCH_SIZE", 2), ("WRITE_SIZE", 1)):
        _write(os.path.join(base, f"{cn}_{raw}", "fa_counter_collection.csv"), CC_HEAD,
               _counter_rows(names, psteps, lambda k, cn=cn, mib=mib: {cn: mib * 1024 / 2}))
        _write(os.path.join(base, f"{cn}_copy", "fa_counter_collection.csv"), CC_HEAD,
               _counter_rows(["__amd_rocclr_copyBuffer"], 3, lambda k, cn=cn: {cn: COPY_MIB * 1024 / 2}))
    cmds = {"kernel_source_sha256": bench.kernel_digest(spec["family"]), "workload": wl, "steps": steps,
            "warmup": 5, "pmc_steps": psteps, "trace": "rocprofv3 --kernel-trace --stats ...",
            "sq": [f"rocprofv3 --pmc pass {i}" for i in range(len(bench.SQ_PASSES))],
            "traffic": ["rocprofv3 --pmc FETCH_SIZE", "copy", "rocprofv3 --pmc WRITE_SIZE", "copy"]}
    with open(os.path.join(base, f"commands_{raw}.json"), "w") as fh:
        json.dump(cmds, fh)
    return spec


@pytest.mark.parametrize("wl", ["0", "1", "2", "3", "4", "fp8", "fp8-causal", "decode", "bwd", "bwd-causal"])
def test_summarize_counters_on_synthetic_output(tmp_path, wl):
    base, out = tmp_path / "prof", tmp_path / "profiles"
    spec = _plant(str(base), wl)
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--summarize-counters", "--workload", wl,
                          "--prof-dir", str(base), "--out-dir", str(out)], capture_output=True, text=True,
                         timeout=120)
    assert res.returncode == 0, res.stderr[-2000:]
    line = json.loads([l for l in res.stdout.splitlines() if l.startswith("{")][-1])
    nk = len(spec["kernels"])
    # 2 MiB read + 1 MiB written per kernel, each counted in 2 KiB units that the copy calibrates exactly
    assert line["hbm_bytes_per_launch"] == pytest.approx(nk * 3 * (1 << 20), rel=1e-9)
    entry = line["counters"]
    derived = [entry] if nk == 1 else list(entry["kernels"].values())
    for d in derived:
        assert d["engine_clock_ghz"] == pytest.approx(CLOCK_GHZ, rel=1e-9)
        assert d["mfma_busy"] == pytest.approx(MFMA_BUSY, rel=1e-9)
        assert d["duration_ms_under_counters"] == pytest.approx(DUR_NS * 1e-6)
        assert d["waves"] == 8192
    for suffix in ("kernel_trace", "sq_counters", "traffic"):
        assert (out / f"{spec['prefix']}_{spec['tag']}_{suffix}.md").exists()
    # both VALU bounds, the second at the planted clock
    sq_md = (out / f"{spec['prefix']}_{spec['tag']}_sq_counters.md").read_text()
    assert sq_md.count("VALU issue bound of") == nk
    if spec["family"] == "fwd":
        assert sq_md.count("One-wave issue bound") == nk and f"at {CLOCK_GHZ:.2f} GHz" in sq_md
    else:
        assert "One-wave issue bound" not in sq_md
    rec = json.load(open(out / os.path.basename(bench._record_path("traffic", spec["family"]))))
    assert rec["workloads"][wl]["algorithmic_bytes_per_launch"] == spec["algo"]
