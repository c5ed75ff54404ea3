"""The counter and traffic records the bench line reports (profiles/*.json,
written by bench.py --collect-counters): used only while the kernel sources
they were taken on are unchanged, and then physically sane."""
import json
import os

import pytest

import bench

WORKLOADS = ["0", "1", "2", "3", "4", "fp8", "fp8-causal", "decode", "bwd", "bwd-causal"]


@pytest.mark.parametrize("wl", WORKLOADS)
def test_records_match_sources_or_are_ignored(wl):
    fam = bench._family(wl)
    path = bench._record_path("traffic", fam)
    rec = json.load(open(path)) if os.path.exists(path) else {}
    current = rec.get("kernel_source_sha256") == bench.kernel_digest(fam)
    entry = rec.get("workloads", {}).get(wl) if current else None
    traffic = bench.traffic_for(wl)
    counters = bench.counters_for(wl, 1.0)
    if entry is None:
        assert traffic is None
        return
    # measured HBM bytes of a call: at least the algorithmic bytes (within the
    # counters' granularity), at most a few times them.  The bound is 8x: a
    # small grid spreads one head's workgroups over the 8 XCDs, and each XCD's
    # L2 then fetches that head's K and V from memory itself (the fp32 L256
    # workload: 8 workgroups, 5.05x).
    algo = entry["algorithmic_bytes_per_launch"]
    assert 0.99 * algo <= traffic <= 8 * algo
    assert counters is not None and counters["hbm_gbps"] == pytest.approx(traffic / 1e-3 / 1e9)
    figures = [counters] + list(counters.get("kernels", {}).values())
    for f in figures:
        for k in ("mfma_busy", "mfma_valu_coexec", "lds_busy"):
            if k in f:
                assert 0.0 <= f[k] <= 1.0
        if f.get("engine_clock_ghz") is not None:
            assert 0.5 < f["engine_clock_ghz"] < 2.6


def test_a_changed_source_voids_the_record(monkeypatch):
    monkeypatch.setattr(bench, "kernel_digest", lambda family="fwd": "0" * 64)
    assert bench.traffic_for("3") is None and bench.counters_for("3", 1.0) is None


def test_valu_bounds_are_ordered():
    """The three VALU issue bounds of a forward record: the chip-wide bound is
    the loosest, one wave at a time the next, one wave beside an MFMA wave
    (slower rates) the tightest; each is the counted instructions at its rates."""
    w = bench._record("counters", "3")
    if w is None:
        pytest.skip("no counter record for the current forward source")
    r = bench.valu_roofline("3", w["duration_ms_under_counters"])
    assert r["frac"] < r["one_wave_frac"] < r["one_wave_beside_mfma_frac"]
    pw = w["per_wave"]
    valu, trans = pw["valu"] - pw["mfma"], pw["v_exp_f32"]
    cyc = (valu - trans) * bench.MFMA_SIDE_VALU_CYCLES + trans * bench.MFMA_SIDE_TRANS_CYCLES
    expect = w["waves"] * cyc / (bench.SIMDS * w["engine_clock_ghz"] * 1e9) * 1e3
    assert r["one_wave_beside_mfma_bound_ms"] == pytest.approx(expect)
