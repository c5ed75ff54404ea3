#!/usr/bin/env python3
"""Benchmark of the exact attention forward pass on one MI355X.

One step = one fa_fwd call over the whole workload (every step of the tiled
online-softmax forward runs inside that one kernel launch).  Default workload:
B=1, H=32, L=8192, d=128, bf16, non-causal, Q and K ~ 3*N(0,1), V ~ N(0,1)
(the long non-causal head-dim-128 case the throughput target is quoted on).

Prints ONE JSON line.  `value` is TFLOP/s counting 4*B*H*L^2*d FLOPs (half for
causal) with inputs resident in HBM before the timed region starts.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import fa_inputs as gen  # noqa: E402

METRIC = "attention fwd TFLOP/s (4·B·H·L²·d) and % of MI355X bf16 MFMA peak"
PEAK_TFLOPS = {gen.BF16: 2516.6, gen.F16: 2516.6, gen.F32: 157.3}   # dense MFMA peaks, MI355X
CSRC = os.path.join(ROOT, "io_aware_tiled_02_amd", "csrc")
# kernel families: the sources their kernels are compiled from (the counter
# and traffic records of a family are keyed to these files' sha256) and the
# name of their record files under profiles/
FAMILIES = {
    "fwd": {"srcs": ("fa_fwd.hip", "fa_device.h"), "record": "fa_fwd_kernel"},
    "splitkv": {"srcs": ("fa_splitkv.hip", "fa_device.h"), "record": "fa_splitkv_kernels"},
    "bwd": {"srcs": ("fa_bwd.hip", "fa_device.h"), "record": "fa_bwd_kernels"},
}


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def _family(workload) -> str:
    w = str(workload)
    return "splitkv" if w == "decode" else "bwd" if w.startswith("bwd") else "fwd"


def kernel_digest(family: str = "fwd") -> str:
    h = hashlib.sha256()
    for n in FAMILIES[family]["srcs"]:
        h.update(open(os.path.join(CSRC, n), "rb").read())
    return h.hexdigest()


def _record_path(kind, family):
    return os.path.join(ROOT, "profiles", f"{kind}_{FAMILIES[family]['record']}.json")


def _record(kind, workload):
    """The workload's entry of a counter or traffic record, if the record was
    taken on the kernel sources of this tree."""
    fam = _family(workload)
    path = _record_path(kind, fam)
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("kernel_source_sha256") != kernel_digest(fam):
        return None
    return rec.get("workloads", {}).get(str(workload))


def traffic_for(workload):
    """Measured HBM bytes of one call (all of its kernels) for a workload
    (0..4, fp8, fp8-causal, decode, bwd, bwd-causal), if the counters were taken
    on the current kernel sources."""
    w = _record("traffic", workload)
    return w["hbm_bytes_per_launch"] if w else None


# VALU issue model of the MI355X SIMD for the softmax roofline: a wave64
# non-transcendental VALU instruction takes 2 SIMD cycles at the chip's fp32
# vector peak (157.3 TFLOP/s = 256 CUs x 4 SIMDs x 2.4 GHz x 32 FMA lanes);
# transcendentals (v_exp_f32, v_log_f32, ...) run at a quarter of that rate.
VALU_CYCLES, TRANS_CYCLES = 2.0, 8.0
SIMDS, ENGINE_GHZ = 1024, 2.4
# One wave's own issue rate, measured on gfx950 (one wave per SIMD issuing
# independent v_fma_f32 / v_add_f32 / v_max3_f32, or v_exp_f32): a wave issues
# a non-transcendental VALU instruction every 5.0 cycles and a transcendental
# every 8.7.  The forward's softmax phases run one wave per SIMD at a time, so
# at this rate, and at the engine clock measured under the counters, they
# bound the kernel from below as well (the "one-wave issue bound").
ONE_WAVE_VALU_CYCLES, ONE_WAVE_TRANS_CYCLES = 5.0, 8.7
# The same wave's rates while the other wave of its SIMD issues MFMAs, as it
# does through every softmax phase of the forward's ping-pong: 5.8 and 9.7
# cycles (measured the same way, beside a wave running back-to-back
# v_mfma_f32_32x32x16_bf16).
MFMA_SIDE_VALU_CYCLES, MFMA_SIDE_TRANS_CYCLES = 5.8, 9.7


def one_wave_bound_ms(waves, valu, trans, clock_ghz, rates=(ONE_WAVE_VALU_CYCLES, ONE_WAVE_TRANS_CYCLES)):
    """All waves' VALU work issued one wave per SIMD at a time at the one-wave
    rates (or the given ones), in ms at `clock_ghz`; None without a clock figure."""
    if not clock_ghz:
        return None
    cycles = (valu - trans) * rates[0] + trans * rates[1]
    return waves * cycles / (SIMDS * clock_ghz * 1e9) * 1e3


def valu_roofline(workload, ms_per_launch):
    """The kernel's VALU work (SQ_INSTS_VALU minus MFMA, SQ_INSTS_VALU_TRANS_F32
    per wave, from the counter record of the current source) priced at the
    issue model above, against the measured launch time: the fraction of the
    VALU issue bound the kernel reaches.  None without a record."""
    w = _record("counters", workload)
    if not w or "per_wave" not in w or not w.get("waves") or not ms_per_launch:
        return None
    pw = w["per_wave"]
    valu = pw["valu"] - pw["mfma"]
    trans = pw["v_exp_f32"]
    cycles = (valu - trans) * VALU_CYCLES + trans * TRANS_CYCLES
    t_ms = w["waves"] * cycles / (SIMDS * ENGINE_GHZ * 1e9) * 1e3
    t1 = one_wave_bound_ms(w["waves"], valu, trans, w.get("engine_clock_ghz"))
    t2 = one_wave_bound_ms(w["waves"], valu, trans, w.get("engine_clock_ghz"),
                           (MFMA_SIDE_VALU_CYCLES, MFMA_SIDE_TRANS_CYCLES))
    return {
        "bound": "alu",
        "achieved": t_ms / ms_per_launch,
        "peak": 1.0,
        "unit": "fraction of the VALU issue bound",
        "frac": t_ms / ms_per_launch,
        "valu_bound_ms": t_ms,
        "valu_per_wave": valu,
        "trans_per_wave": trans,
        "waves": w["waves"],
        "model": f"non-transcendental VALU {VALU_CYCLES:g} and transcendental {TRANS_CYCLES:g} SIMD cycles per "
                 f"wave64 instruction, {SIMDS} SIMDs at {ENGINE_GHZ} GHz",
        "one_wave_bound_ms": t1,
        "one_wave_frac": None if t1 is None else t1 / ms_per_launch,
        "one_wave_model": f"the same VALU work issued one wave per SIMD at a time, {ONE_WAVE_VALU_CYCLES:g} / "
                          f"{ONE_WAVE_TRANS_CYCLES:g} cycles per instruction (measured one-wave rates), at the engine "
                          "clock measured under the counters",
        "one_wave_beside_mfma_bound_ms": t2,
        "one_wave_beside_mfma_frac": None if t2 is None else t2 / ms_per_launch,
        "one_wave_beside_mfma_model": f"as the one-wave bound, at {MFMA_SIDE_VALU_CYCLES:g} / "
                                      f"{MFMA_SIDE_TRANS_CYCLES:g} cycles per instruction (one wave's measured rates "
                                      "while the other wave of its SIMD issues MFMAs)",
    }


def counters_for(workload, ms_per_launch):
    """SQ-counter figures of the workload's kernels (rocprofv3 --pmc runs made by
    --collect-counters), if they were taken on the current kernel sources; with
    the achieved HBM rate of this run when the traffic record exists."""
    w = _record("counters", workload)
    if not w:
        return None
    keys = ("mfma_busy", "mfma_valu_coexec", "lds_busy", "lds_bank_conflict_cycles", "engine_clock_ghz",
            "duration_ms_under_counters", "hbm_gbps_under_counters")
    out = {k: w[k] for k in keys if k in w}
    if "kernels" in w:
        out["kernels"] = {n: {k: v[k] for k in keys if k in v} for n, v in w["kernels"].items()}
    out["summary"] = w.get("summary")
    traffic = traffic_for(workload)
    if traffic is not None and ms_per_launch:
        out["hbm_gbps"] = traffic / (ms_per_launch * 1e-3) / 1e9
    return out


def cpu_baseline(cfg, q, k, v, target_s: float):
    """The fp64 oracle timed on this host's cores over a bounded sample of query rows."""
    import oracle
    nth = oracle.max_threads()
    per_row = 4.0 * cfg.L * cfg.d * (0.5 if cfg.causal else 1.0)   # metric FLOPs of one query row
    rows0 = gen.sample_rows(cfg.L, min(128, cfg.L), cfg.seed)
    t = time.perf_counter()
    oracle.fwd(q, k, v, cfg.dtype, cfg.scale, cfg.causal, rows0)
    t0 = max(time.perf_counter() - t, 1e-3)
    nrows = int(min(cfg.L, max(16, rows0.size * target_s / t0)))
    rows = gen.sample_rows(cfg.L, nrows, cfg.seed)
    t = time.perf_counter()
    oracle.fwd(q, k, v, cfg.dtype, cfg.scale, cfg.causal, rows)
    dt = time.perf_counter() - t
    flops = per_row * rows.size * cfg.B * cfg.H
    return {
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": nth,
        "kind": "oracle",
        "sample": (f"{rows.size} query rows per head x {cfg.B * cfg.H} heads of the same workload "
                   f"(all L={cfg.L} keys each), fp64 C oracle, OpenMP; {dt:.1f} s"),
        "seconds": dt,
        "cpu_model": _cpu_model(),
        "nproc": os.cpu_count(),
    }


def _cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline_decode(cfg, q, k, v, target_s: float):
    """The fp64 oracle (key-range attention over all keys) on a bounded sample of heads."""
    import oracle
    nth = oracle.max_threads()
    bh = cfg.B * cfg.H
    qs = q.reshape(bh, 1, cfg.Lq, cfg.d)
    ks = k.reshape(bh, 1, cfg.Lk, cfg.d)
    vs = v.reshape(bh, 1, cfg.Lk, cfg.d)
    t = time.perf_counter()
    oracle.attn_range(qs[:2], ks[:2], vs[:2], cfg.dtype, cfg.scale, 0, cfg.Lk)
    t0 = max(time.perf_counter() - t, 1e-3)
    nh = int(min(bh, max(2, 2 * target_s / t0)))
    t = time.perf_counter()
    oracle.attn_range(qs[:nh], ks[:nh], vs[:nh], cfg.dtype, cfg.scale, 0, cfg.Lk)
    dt = time.perf_counter() - t
    eb = 4 if cfg.dtype == gen.F32 else 2
    nbytes = nh * (2 * cfg.Lq + 2 * cfg.Lk) * cfg.d * eb + 4 * nh * cfg.Lq
    return {
        "value": nbytes / dt / 1e9,
        "unit": "GB/s",
        "cores": min(nth, cfg.Lq),          # the oracle's threads split query rows of one head
        "kind": "oracle",
        "sample": (f"{nh} of {bh} (b, h) heads of the same workload, each {cfg.Lq} query row(s) against all "
                   f"{cfg.Lk} keys, fp64 C oracle (OpenMP over query rows); {dt:.1f} s"),
        "seconds": dt,
        "cpu_model": _cpu_model(),
        "nproc": os.cpu_count(),
    }


def bench_decode(args, torch, fa):
    """Split-K/V attention (fa_fwd_splitkv: chunk kernel + merge) on the decoding shape."""
    cfg = gen.DECODE
    log(f"[bench] decode: {cfg.name}; generating inputs")
    q, k, v = gen.make_decode_qkv(cfg)

    def dev(a):
        if cfg.dtype == gen.BF16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to("cuda")
        return torch.from_numpy(a).to("cuda")

    qd, kd, vd = dev(q), dev(k), dev(v)
    o = torch.empty_like(qd)
    lse = torch.empty((cfg.B, cfg.H, cfg.Lq), dtype=torch.float32, device="cuda")
    nsplit = fa.fa_splitkv_splits(cfg.B, cfg.H, cfg.Lk)
    need = fa.fa_splitkv_workspace_bytes(cfg.B, cfg.H, cfg.Lq, cfg.Lk, cfg.d, nsplit)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    call = (qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), o.data_ptr(), lse.data_ptr(), cfg.B, cfg.H, cfg.Lq,
            cfg.Lk, cfg.d, float(cfg.scale), cfg.dtype, nsplit, ws.data_ptr(), need, stream.cuda_stream)
    log(f"[bench] warmup {args.warmup} (nsplit {nsplit})")
    for _ in range(args.warmup):
        rc = fa.fa_fwd_splitkv(*call)
        if rc != 0:
            raise SystemExit(f"fa_fwd_splitkv failed: {rc} {fa.fa_strerror(rc)}")
    torch.cuda.synchronize()
    log(f"[bench] timing {args.steps} steps")
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for _ in range(args.steps):
        fa.fa_fwd_splitkv(*call)
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / args.steps
    gbs = cfg.algorithmic_bytes / (ms * 1e-3) / 1e9
    log(f"[bench] {ms:.4f} ms/step, {gbs:.0f} GB/s ({100 * gbs / 8000:.1f}% of 8000 GB/s)")
    out = {
        "metric": "split-K/V decode: algorithmic HBM GB/s (Q, K, V read once; O, lse written once)",
        "value": gbs,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": gen.DTYPE_NAMES[cfg.dtype],
        "data": "synthetic (seeded SplitMix64 + Box-Muller normals)",
        "config": {"workload": cfg.name, "B": cfg.B, "H": cfg.H, "Lq": cfg.Lq, "Lk": cfg.Lk, "d": cfg.d,
                   "scale": cfg.scale, "nsplit": nsplit, "tflops": cfg.flops / (ms * 1e-3) / 1e12},
        "roofline": {
            "bound": "hbm",
            "achieved": gbs,
            "peak": 8000.0,
            "unit": "GB/s",
            "frac": gbs / 8000.0,
            "traffic": traffic_for("decode"),
            "kernel": "fa_splitkv_kernel + fa_combine_kernel (one fa_fwd_splitkv call)",
            "algorithmic_bytes_per_launch": cfg.algorithmic_bytes,
            "avg_launch_ms": ms,
        },
        "counters": counters_for("decode", ms),
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        log("[bench] CPU baseline (fp64 oracle on a sample of heads)")
        out["cpu_baseline"] = cpu_baseline_decode(cfg, q, k, v, args.cpu_seconds)
    print(json.dumps(out), flush=True)


def cpu_baseline_bwd(cfg, q, k, v, g, target_s: float):
    """The fp64 oracle's gradients for whole heads of the same workload (bounded sample)."""
    import oracle
    nth = oracle.max_threads()
    bh = cfg.B * cfg.H
    sl = lambda a, n: a.reshape(bh, cfg.L, cfg.d)[:n][None]
    t = time.perf_counter()
    oracle.bwd(sl(q, 1), sl(k, 1), sl(v, 1), sl(g, 1), cfg.dtype, cfg.scale, cfg.causal)
    dt = time.perf_counter() - t
    nh = 1
    if dt < target_s / 2:
        nh = int(min(bh, max(1, target_s / dt)))
        t = time.perf_counter()
        oracle.bwd(sl(q, nh), sl(k, nh), sl(v, nh), sl(g, nh), cfg.dtype, cfg.scale, cfg.causal)
        dt = time.perf_counter() - t
    flops = cfg.flops * nh / bh
    return {
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": nth,
        "kind": "oracle",
        "sample": f"{nh} of {bh} heads of the same workload (every row), fp64 C oracle, OpenMP; {dt:.1f} s",
        "seconds": dt,
        "cpu_model": _cpu_model(),
        "nproc": os.cpu_count(),
    }


def bench_bwd(args, torch, fa, cfg):
    """The backward pass (fa_bwd: D, dK/dV, dQ kernels) after one forward pass for o and lse."""
    log(f"[bench] backward: {cfg.name}; generating inputs")
    q, k, v, g = gen.make_bwd_inputs(cfg)

    def dev(a):
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to("cuda")

    qd, kd, vd, gd = (dev(x) for x in (q, k, v, g))
    B, H, L, d = cfg.B, cfg.H, cfg.L, cfg.d
    o = torch.empty_like(qd)
    lse = torch.empty((B, H, L), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    rc = fa.fa_fwd(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), o.data_ptr(), lse.data_ptr(), B, H, L, d,
                   float(cfg.scale), cfg.causal, cfg.dtype, stream.cuda_stream)
    if rc != 0:
        raise SystemExit(f"fa_fwd failed: {rc} {fa.fa_strerror(rc)}")
    dq, dk, dv = torch.empty_like(qd), torch.empty_like(kd), torch.empty_like(vd)
    need = fa.fa_bwd_workspace_bytes(B, H, L)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    call = (qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), o.data_ptr(), lse.data_ptr(), gd.data_ptr(),
            dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, L, d, float(cfg.scale), cfg.causal, cfg.dtype,
            ws.data_ptr(), need, stream.cuda_stream)
    log(f"[bench] warmup {args.warmup}")
    for _ in range(args.warmup):
        rc = fa.fa_bwd(*call)
        if rc != 0:
            raise SystemExit(f"fa_bwd failed: {rc} {fa.fa_strerror(rc)}")
    torch.cuda.synchronize()
    log(f"[bench] timing {args.steps} steps")
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for _ in range(args.steps):
        fa.fa_bwd(*call)
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / args.steps
    tflops = cfg.flops / (ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[cfg.dtype]
    log(f"[bench] {ms:.4f} ms/step, {tflops:.1f} TFLOP/s ({100 * tflops / peak:.1f}% of {peak})")
    out = {
        "metric": "attention bwd TFLOP/s (10*B*H*L^2*d: S, dP, dV, dK, dQ products; half for causal) "
                  "and % of MI355X bf16 MFMA peak",
        "value": tflops,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": gen.DTYPE_NAMES[cfg.dtype],
        "data": "synthetic (seeded SplitMix64 + Box-Muller normals)",
        "config": {"workload": cfg.name, "B": B, "H": H, "L": L, "d": d, "causal": bool(cfg.causal),
                   "scale": cfg.scale, "pct_of_peak": 100.0 * tflops / peak},
        "roofline": {
            "bound": "mfma",
            "achieved": tflops,
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": tflops / peak,
            "traffic": traffic_for(args.workload),
            "kernel": "fa_bwd_pre_kernel + fa_bwd_dq_kernel + fa_bwd_dkdv_kernel (one fa_bwd call)",
            "per_launch_flops": cfg.flops,
            "avg_launch_ms": ms,
            "algorithmic_bytes_per_launch": cfg.algorithmic_bytes,
        },
        "counters": counters_for(args.workload, ms),
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        log("[bench] CPU baseline (fp64 oracle gradients on whole heads)")
        out["cpu_baseline"] = cpu_baseline_bwd(cfg, q, k, v, g, args.cpu_seconds)
    print(json.dumps(out), flush=True)


# Peak of the FP8 forward's MFMA work: half its FLOPs (S = Q K^T) run on E4M3
# operands (5.0 PFLOP/s dense on MI355X), half (P V) on 16-bit ones (2.5166),
# so at both peaks a launch takes F/2/5000 + F/2/2516.6 and the combined peak is
# the harmonic mean 2 / (1/5000 + 1/2516.6).
FP8_MIXED_PEAK = 2.0 / (1.0 / 5000.0 + 1.0 / 2516.6)


def cpu_baseline_fp8(cfg, q, k, v, target_s: float):
    """The oracle (quantiser, then attention on the quantised Q, K) on a bounded
    sample of query rows of every head."""
    import oracle
    nth = oracle.max_threads()
    per_row = 4.0 * cfg.L * cfg.d * (0.5 if cfg.causal else 1.0)
    t = time.perf_counter()
    q8, sq = oracle.quantize_fp8(q, cfg.dtype, cfg.block_q)
    k8, sk = oracle.quantize_fp8(k, cfg.dtype, cfg.block_k)
    tq = time.perf_counter() - t
    rows0 = gen.sample_rows(cfg.L, min(64, cfg.L), cfg.seed)
    t = time.perf_counter()
    oracle.fwd_fp8(q8, k8, sq, sk, v, cfg.dtype, cfg.scale, cfg.causal, cfg.block_q, cfg.block_k, rows0)
    t0 = max(time.perf_counter() - t, 1e-3)
    nrows = int(min(cfg.L, max(16, rows0.size * target_s / t0)))
    rows = gen.sample_rows(cfg.L, nrows, cfg.seed)
    t = time.perf_counter()
    oracle.fwd_fp8(q8, k8, sq, sk, v, cfg.dtype, cfg.scale, cfg.causal, cfg.block_q, cfg.block_k, rows)
    dt = time.perf_counter() - t
    flops = per_row * rows.size * cfg.B * cfg.H
    return {
        "value": flops / (dt + tq * rows.size / cfg.L) / 1e12,
        "unit": "TFLOP/s",
        "cores": nth,
        "kind": "oracle",
        "sample": (f"quantisation of all of Q and K ({tq:.1f} s, charged pro rata), then {rows.size} query rows "
                   f"per head x {cfg.B * cfg.H} heads (all L={cfg.L} keys each), fp64 C oracle, OpenMP; "
                   f"{dt:.1f} s"),
        "seconds": dt,
        "cpu_model": _cpu_model(),
        "nproc": os.cpu_count(),
    }


def bench_fp8(args, torch, fa, cfg):
    """The FP8 forward: one step quantises Q and K (fa_quantize_fp8, two
    launches) and runs fa_fwd_fp8 on the codes and the 16-bit V."""
    log(f"[bench] fp8: {cfg.name}; generating inputs")
    q, k, v = gen.make_fp8_inputs(cfg)

    def dev(a):
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to("cuda")

    qd, kd, vd = (dev(x) for x in (q, k, v))
    B, H, L, d = cfg.B, cfg.H, cfg.L, cfg.d
    q8 = torch.empty(qd.shape, dtype=torch.uint8, device="cuda")
    k8 = torch.empty_like(q8)
    sq = torch.empty((B * H, (L + cfg.block_q - 1) // cfg.block_q), dtype=torch.float32, device="cuda")
    sk = torch.empty((B * H, (L + cfg.block_k - 1) // cfg.block_k), dtype=torch.float32, device="cuda")
    o = torch.empty_like(vd)
    lse = torch.empty((B, H, L), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    quant_q = (qd.data_ptr(), cfg.dtype, B, H, L, d, cfg.block_q, q8.data_ptr(), sq.data_ptr(), sh)
    quant_k = (kd.data_ptr(), cfg.dtype, B, H, L, d, cfg.block_k, k8.data_ptr(), sk.data_ptr(), sh)
    attn = (q8.data_ptr(), k8.data_ptr(), sq.data_ptr(), sk.data_ptr(), vd.data_ptr(), o.data_ptr(), lse.data_ptr(),
            B, H, L, d, float(cfg.scale), cfg.causal, cfg.dtype, cfg.block_q, cfg.block_k, sh)

    def step():
        rc = fa.fa_quantize_fp8(*quant_q) or fa.fa_quantize_fp8(*quant_k) or fa.fa_fwd_fp8(*attn)
        if rc != 0:
            raise SystemExit(f"FP8 step failed: {rc} {fa.fa_strerror(rc)}")

    log(f"[bench] warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    log(f"[bench] timing {args.steps} steps")
    ev[0].record(stream)
    for _ in range(args.steps):
        step()
    ev[1].record(stream)
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[1]) / args.steps
    # the attention kernel alone, same inputs, same stream
    ev[2].record(stream)
    for _ in range(args.steps):
        fa.fa_fwd_fp8(*attn)
    ev[3].record(stream)
    torch.cuda.synchronize()
    ms_attn = ev[2].elapsed_time(ev[3]) / args.steps
    tflops = cfg.flops / (ms * 1e-3) / 1e12
    tflops_attn = cfg.flops / (ms_attn * 1e-3) / 1e12
    peak = FP8_MIXED_PEAK
    log(f"[bench] step {ms:.4f} ms ({tflops:.1f} TFLOP/s); attention kernel {ms_attn:.4f} ms "
        f"({tflops_attn:.1f} TFLOP/s, {100 * tflops_attn / peak:.1f}% of the {peak:.0f} mixed FP8/bf16 peak)")
    out = {
        "metric": "attention fwd TFLOP/s (4*B*H*L^2*d) with Q, K block-quantised to FP8 E4M3 (quantisation "
                  "included) and % of the mixed FP8/bf16 MFMA peak",
        "value": tflops,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "e4m3 (Q, K) + bf16 (V, P)",
        "data": "synthetic (seeded SplitMix64 + Box-Muller normals)",
        "config": {"workload": cfg.name, "B": B, "H": H, "L": L, "d": d, "causal": bool(cfg.causal),
                   "scale": cfg.scale, "sigma_qkv": [cfg.sigma_q, cfg.sigma_k, cfg.sigma_v],
                   "block_q": cfg.block_q, "block_k": cfg.block_k,
                   "attention_kernel_ms": ms_attn, "quantise_ms": ms - ms_attn},
        "roofline": {
            "bound": "mfma",
            "achieved": tflops_attn,
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": tflops_attn / peak,
            "traffic": traffic_for(args.workload),
            "kernel": "fa_fwd_h_kernel (FP8 scores)",
            "per_launch_flops": cfg.flops,
            "avg_launch_ms": ms_attn,
        },
        "roofline_valu": valu_roofline(args.workload, ms_attn),
        "counters": counters_for(args.workload, ms_attn),
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        log("[bench] CPU baseline (oracle quantiser + attention on a sample of rows)")
        out["cpu_baseline"] = cpu_baseline_fp8(cfg, q, k, v, args.cpu_seconds)
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    # the engine clock ramps up over the first ~0.1 s of load: 100 untimed steps
    # (about 0.1 s of the bench workload) reach the steady-state rate
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default="3",
                    help="workload index 0..4 (default 3); 'decode' (split-K/V decoding shape); "
                         "'bwd' / 'bwd-causal' (backward pass shapes); 'fp8' / 'fp8-causal' (FP8 forward)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target length of the CPU-baseline run")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--collect-counters", action="store_true",
                    help="run rocprofv3 (kernel trace, SQ counter passes, FETCH/WRITE_SIZE against a plain copy) "
                         "on this workload as child processes; write the summaries and records under profiles/")
    ap.add_argument("--summarize-counters", action="store_true",
                    help="only the summary step of --collect-counters, from raw output already under --prof-dir")
    ap.add_argument("--prof-dir", default=os.path.join(ROOT, "prof_raw"),
                    help="where --collect-counters keeps rocprofv3's raw output")
    ap.add_argument("--out-dir", default=os.path.join(ROOT, "profiles"),
                    help="where the counter summaries and records are written")
    ap.add_argument("--counter-timeout", type=float, default=240.0, help="time limit of each rocprofv3 run (s)")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB (counter calibration) and exit")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: this library has no multi-GPU path "
              "(each GPU would run the same kernel on its own heads); use --gpus 1", file=sys.stderr)
        sys.exit(2)

    if args.collect_counters:                 # child processes only; this one stays off the GPU
        return collect_counters(args)
    if args.summarize_counters:
        return summarize_counters(args)

    import torch
    import io_aware_tiled_02_amd as fa

    if args.copy_probe:
        # A plain copy of known size: FETCH_SIZE / WRITE_SIZE read on it give
        # the factor between those counters and bytes actually moved.
        n = args.copy_probe << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        src.fill_(1)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": n, "launches": 3}), flush=True)
        return

    if args.workload == "decode":
        return bench_decode(args, torch, fa)
    if args.workload in ("bwd", "bwd-causal"):
        return bench_bwd(args, torch, fa, gen.BWD[0 if args.workload == "bwd" else 1])
    if args.workload in ("fp8", "fp8-causal"):
        return bench_fp8(args, torch, fa, gen.FP8[0 if args.workload == "fp8" else 1])
    cfg = gen.config(int(args.workload))
    log(f"[bench] workload {cfg.index}: {cfg.name}; generating inputs")
    q, k, v = gen.make_qkv(cfg)

    def dev(a):
        if cfg.dtype == gen.BF16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to("cuda")
        return torch.from_numpy(a).to("cuda")

    qd, kd, vd = dev(q), dev(k), dev(v)
    o = torch.empty_like(qd)
    lse = torch.empty((cfg.B, cfg.H, cfg.L), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    call = (qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), o.data_ptr(), lse.data_ptr(),
            cfg.B, cfg.H, cfg.L, cfg.d, float(cfg.scale), cfg.causal, cfg.dtype, sh)

    log(f"[bench] warmup {args.warmup}")
    for _ in range(args.warmup):
        rc = fa.fa_fwd(*call)
        if rc != 0:
            raise SystemExit(f"fa_fwd failed: {rc} {fa.fa_strerror(rc)}")
    torch.cuda.synchronize()

    log(f"[bench] timing {args.steps} steps")
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        fa.fa_fwd(*call)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = ev0.elapsed_time(ev1) / args.steps
    tflops = cfg.flops / (ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[cfg.dtype]
    log(f"[bench] {ms:.4f} ms/step, {tflops:.1f} TFLOP/s ({100 * tflops / peak:.1f}% of {peak} TFLOP/s); "
        f"wall {wall:.3f} s")

    br, bc, wgs = fa.fa_fwd_tiling(cfg.B, cfg.H, cfg.L, cfg.d, cfg.causal, cfg.dtype)
    traffic = traffic_for(cfg.index)
    roofline = {
        "bound": "mfma",
        "achieved": tflops,
        "peak": peak,
        "unit": "TFLOP/s",
        "frac": tflops / peak,
        "traffic": traffic,
        "kernel": "fa_fwd_h_kernel" if cfg.dtype != gen.F32 else "fa_fwd_f32_kernel",
        "per_launch_flops": cfg.flops,
        "avg_launch_ms": ms,
        "algorithmic_bytes_per_launch": cfg.algorithmic_bytes,
    }
    out = {
        "metric": METRIC,
        "value": tflops,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": gen.DTYPE_NAMES[cfg.dtype],
        "data": "synthetic (seeded SplitMix64 + Box-Muller normals, not torch.randn)",
        "config": {
            "workload": cfg.name,
            "B": cfg.B, "H": cfg.H, "L": cfg.L, "d": cfg.d,
            "causal": bool(cfg.causal),
            "scale": cfg.scale,
            "sigma_qkv": [cfg.sigma_q, cfg.sigma_k, cfg.sigma_v],
            "block_rows": br, "block_cols": bc, "workgroups": wgs,
            "pct_of_peak": 100.0 * tflops / peak,
        },
        "roofline": roofline,
        "roofline_valu": valu_roofline(cfg.index, ms),
        "counters": counters_for(cfg.index, ms),
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        log("[bench] CPU baseline (fp64 oracle on a sample of rows)")
        out["cpu_baseline"] = cpu_baseline(cfg, q, k, v, args.cpu_seconds)
    print(json.dumps(out), flush=True)


# ---- rocprofv3 counter collection (--collect-counters) ----
# This mode never touches the GPU itself: every run is a child process,
# rocprofv3 -- python3 bench.py ..., one counter pass per run (at most 8 SQ,
# 2 GRBM and one of FETCH_SIZE / WRITE_SIZE each).
XCDS, CUS, SIMDS_PER_CU = 8, 256, 4          # MI355X
SQ_PASSES = [
    ["SQ_WAVES", "SQ_BUSY_CYCLES", "SQ_WAVE_CYCLES", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_VALU_MFMA_COEXEC_CYCLES",
     "SQ_INSTS_MFMA", "SQ_INSTS_VALU", "SQ_INSTS_LDS"],
    ["SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE", "SQ_WAIT_INST_LDS", "SQ_WAIT_ANY", "SQ_ACTIVE_INST_VALU",
     "SQ_ACTIVE_INST_LDS", "SQ_LDS_ADDR_CONFLICT", "SQ_WAIT_INST_ANY"],
    ["GRBM_GUI_ACTIVE", "SQ_BUSY_CU_CYCLES", "SQ_INSTS_SALU", "SQ_ACTIVE_INST_ANY", "SQ_INSTS_VALU_TRANS_F32",
     "SQ_LDS_DATA_FIFO_FULL", "SQ_INSTS_LDS_LOAD_BANDWIDTH", "SQ_LDS_UNALIGNED_STALL"],
]
COPY_MIB = 512


def _workload_spec(wl):
    """What --collect-counters profiles for a bench workload: its kernel family,
    file tag and title, the kernels of one call (name substrings), their FLOPs
    per launch, and the algorithmic bytes of one call."""
    def causal_s(c):
        return "causal" if c.causal else "non-causal"
    if wl.isdigit():
        c = gen.config(int(wl))
        k = "fa_fwd_f32_kernel" if c.dtype == gen.F32 else "fa_fwd_h_kernel"
        return dict(family="fwd", prefix=k, kernels=[k], flops={k: c.flops}, algo=c.algorithmic_bytes,
                    tag=f"{gen.DTYPE_NAMES[c.dtype]}_d{c.d}_L{c.L}" + ("_causal" if c.causal else ""),
                    title=f"{gen.DTYPE_NAMES[c.dtype]}, B={c.B} H={c.H} L={c.L} d={c.d}, {causal_s(c)}",
                    algo_what="Q, K, V read once, O and lse written once")
    if wl in ("fp8", "fp8-causal"):
        c = gen.FP8[0 if wl == "fp8" else 1]
        k = "fa_fwd_h_kernel"
        return dict(family="fwd", prefix=k, kernels=[k], flops={k: c.flops}, algo=c.algorithmic_bytes,
                    tag=f"fp8_d{c.d}_L{c.L}" + ("_causal" if c.causal else ""),
                    title=f"FP8 scores, B={c.B} H={c.H} L={c.L} d={c.d}, {causal_s(c)}",
                    algo_what="E4M3 codes of Q and K, their float32 block scales and V read once, O and lse "
                              "written once")
    if wl == "decode":
        c = gen.DECODE
        ks = ["fa_splitkv_kernel", "fa_combine_kernel"]
        return dict(family="splitkv", prefix="fa_splitkv_kernels", kernels=ks, flops={}, algo=c.algorithmic_bytes,
                    tag=f"{gen.DTYPE_NAMES[c.dtype]}_d{c.d}_decode_Lk{c.Lk}",
                    title=f"{gen.DTYPE_NAMES[c.dtype]} decode, B={c.B} H={c.H} Lq={c.Lq} Lk={c.Lk} d={c.d}",
                    algo_what="Q, K, V read once, O and lse written once")
    if wl in ("bwd", "bwd-causal"):
        c = gen.BWD[0 if wl == "bwd" else 1]
        ks = ["fa_bwd_dkdv_kernel", "fa_bwd_dq_kernel", "fa_bwd_pre_kernel"]
        # dK/dV forms S, dP, dV, dK (4 of the 5 products); dQ forms S, dP, dQ
        return dict(family="bwd", prefix="fa_bwd_kernels", kernels=ks,
                    flops={ks[0]: c.flops * 4 // 5, ks[1]: c.flops * 3 // 5, ks[2]: 0}, algo=c.algorithmic_bytes,
                    tag=f"{gen.DTYPE_NAMES[c.dtype]}_d{c.d}_L{c.L}" + ("_causal" if c.causal else ""),
                    title=f"backward, {gen.DTYPE_NAMES[c.dtype]}, B={c.B} H={c.H} L={c.L} d={c.d}, {causal_s(c)}",
                    algo_what="Q, K, V, O, dO and lse read once, dQ, dK, dV written once")
    raise SystemExit("--collect-counters takes a bench workload: 0..4, fp8, fp8-causal, decode, bwd, bwd-causal")


def _rocprof(cmd_args, outdir, child, timeout_s):
    """One rocprofv3 run of `child` (a bench.py command line); returns the command string."""
    import subprocess
    os.makedirs(outdir, exist_ok=True)
    cmd = ["rocprofv3", *cmd_args, "-d", outdir, "-o", "fa", "--output-format", "csv", "--",
           sys.executable, os.path.join(ROOT, "bench.py"), *child]
    env = dict(os.environ, TMPDIR="/tmp")
    shown = "cd /tmp && export TMPDIR=/tmp && " + " ".join(
        c.replace(ROOT, "$REPO").replace(sys.executable, "python3") for c in cmd)
    print(f"[counters] {shown}", flush=True)
    res = subprocess.run(cmd, cwd="/tmp", env=env, capture_output=True, text=True, timeout=timeout_s)
    ok_line = any(l.startswith("{") for l in res.stdout.splitlines())
    # rocprofv3 may end with SIGSEGV after the program finished and its files are whole
    if res.returncode != 0 and not (res.returncode in (139, -11) and ok_line):
        sys.stderr.write(res.stdout[-3000:] + res.stderr[-3000:])
        raise SystemExit(f"rocprofv3 run failed with status {res.returncode}")
    return shown


def _csv_rows(outdir, suffix):
    import csv
    import glob
    rows = []
    for f in sorted(glob.glob(os.path.join(outdir, "**", f"*{suffix}"), recursive=True)):
        with open(f, newline="") as fh:
            rows.extend(csv.DictReader(fh))
    if not rows:
        raise SystemExit(f"no *{suffix} under {outdir}")
    return rows


def _col(row, *names):
    for n in names:
        if n in row and row[n] != "":
            return row[n]
    raise KeyError(f"none of {names} in {sorted(row)}")


def _counter_means(outdir, name_pred, last):
    """Mean per dispatch over the last `last` dispatches of the kernels whose
    name satisfies name_pred: ({counter: mean}, kernel name, dispatches)."""
    per = {}
    kname = None
    for r in _csv_rows(outdir, "counter_collection.csv"):
        name = _col(r, "Kernel_Name", "Kernel-Name", "KernelName")
        if not name_pred(name):
            continue
        kname = name
        did = int(_col(r, "Dispatch_Id", "Dispatch-Id", "Correlation_Id"))
        cn = _col(r, "Counter_Name", "Counter-Name")
        per.setdefault(did, {})
        per[did][cn] = per[did].get(cn, 0.0) + float(_col(r, "Counter_Value", "Counter-Value"))
    if not per:
        raise SystemExit(f"no matching kernel in the counter files under {outdir}")
    ids = sorted(per)[-last:]
    names = set().union(*(per[i] for i in ids))
    return {c: sum(per[i].get(c, 0.0) for i in ids) / len(ids) for c in names}, kname, len(ids)


def _trace_durations_ns(outdir, name_pred, last):
    rows = [r for r in _csv_rows(outdir, "kernel_trace.csv") if name_pred(_col(r, "Kernel_Name", "Kernel-Name"))]
    rows.sort(key=lambda r: int(_col(r, "Start_Timestamp", "Start-Timestamp")))
    d = [int(_col(r, "End_Timestamp", "End-Timestamp")) - int(_col(r, "Start_Timestamp", "Start-Timestamp"))
         for r in rows]
    return d[-last:], len(d)


def _merge_record(path, sha, workload, entry, extra=None):
    rec = json.load(open(path)) if os.path.exists(path) else {}
    if rec.get("kernel_source_sha256") != sha:
        rec = {"kernel_source_sha256": sha, "workloads": {}}     # records of another source are dropped
    rec.update(extra or {})
    rec.setdefault("workloads", {})[str(workload)] = entry
    with open(path, "w") as fh:
        json.dump(rec, fh, indent=1)


def collect_counters(args):
    """Run the rocprofv3 passes on the workload's kernels (child processes; raw
    output under --prof-dir, with a record of the commands), then summarise them
    (summarize_counters)."""
    wl = args.workload
    spec = _workload_spec(wl)
    tag = spec["tag"]
    raw = f"{spec['prefix']}_{tag}"               # raw output directories of this workload
    base = os.path.abspath(args.prof_dir)
    T = args.counter_timeout
    warm = args.warmup
    child = ["--workload", wl, "--steps", "3", "--warmup", str(warm), "--no-cpu-baseline"]
    cmds = {"kernel_source_sha256": kernel_digest(spec["family"]), "workload": wl, "steps": args.steps,
            "warmup": warm, "pmc_steps": 3}
    # 1. kernel trace with the bench's own step count
    cmds["trace"] = _rocprof(["--kernel-trace", "--stats"], os.path.join(base, f"kt_{raw}"),
                             ["--workload", wl, "--steps", str(args.steps), "--warmup", str(warm),
                              "--no-cpu-baseline"], T)
    # 2. SQ counter passes (the GRBM pass also records the kernel trace, for the clock)
    cmds["sq"] = []
    for i, counters in enumerate(SQ_PASSES):
        extra = ["--kernel-trace"] if "GRBM_GUI_ACTIVE" in counters else []
        cmds["sq"].append(_rocprof(["--pmc", *counters, *extra], os.path.join(base, f"sq{i}_{raw}"), child, T))
    # 3. HBM traffic: FETCH_SIZE and WRITE_SIZE on the kernels and on a plain copy of known size
    cmds["traffic"] = []
    for cn in ("FETCH_SIZE", "WRITE_SIZE"):
        cmds["traffic"].append(_rocprof(["--pmc", cn], os.path.join(base, f"{cn}_{raw}"), child, T))
        cmds["traffic"].append(_rocprof(["--pmc", cn], os.path.join(base, f"{cn}_copy"),
                                        ["--copy-probe", str(COPY_MIB)], T))
    with open(os.path.join(base, f"commands_{raw}.json"), "w") as fh:
        json.dump(cmds, fh, indent=1)
    return summarize_counters(args)


def summarize_counters(args):
    """Derived figures from the raw rocprofv3 output of collect_counters (no GPU
    needed): writes the kernel-trace, SQ-counter and traffic summaries and the
    records the bench line reports, under --out-dir."""
    wl = args.workload
    spec = _workload_spec(wl)
    tag, title, fam = spec["tag"], spec["title"], spec["family"]
    raw = f"{spec['prefix']}_{tag}"
    base = os.path.abspath(args.prof_dir)
    cmds = json.load(open(os.path.join(base, f"commands_{raw}.json")))
    sha = cmds["kernel_source_sha256"]
    if sha != kernel_digest(fam):
        raise SystemExit("the raw counters were taken on another kernel source than the one in this tree")
    steps, warm, psteps = cmds["steps"], cmds["warmup"], cmds["pmc_steps"]
    pdir = os.path.abspath(args.out_dir)
    os.makedirs(pdir, exist_ok=True)
    preds = {k: (lambda n, k=k: k in n) for k in spec["kernels"]}
    srcs = " then ".join(FAMILIES[fam]["srcs"])

    kt = os.path.join(base, f"kt_{raw}")
    stats_rows = _csv_rows(kt, "kernel_stats.csv")
    per = {}
    for k in spec["kernels"]:
        st = [r for r in stats_rows if preds[k](_col(r, "Name"))][0]
        durs, ncalls = _trace_durations_ns(kt, preds[k], steps)
        sq = {}
        for i in range(len(SQ_PASSES)):
            sq.update(_counter_means(os.path.join(base, f"sq{i}_{raw}"), preds[k], psteps)[0])
        pmc_durs, _ = _trace_durations_ns(os.path.join(base, f"sq{len(SQ_PASSES) - 1}_{raw}"), preds[k], psteps)
        per[k] = dict(name=_col(st, "Name"), st=st, durs=durs, ncalls=ncalls, sq=sq, pmc_durs=pmc_durs)
    traffic, calib = {}, {}
    copy_pred = lambda n: "copy" in n.lower() and "fill" not in n.lower()   # noqa: E731
    for cn in ("FETCH_SIZE", "WRITE_SIZE"):
        cv, cname, ncp = _counter_means(os.path.join(base, f"{cn}_copy"), copy_pred, 3)
        factor = (COPY_MIB << 20) / (cv[cn] * 1024.0)
        calib[cn] = dict(copy_kib=cv[cn], copy_n=ncp, factor=factor, copy_kernel=cname)
        for k in spec["kernels"]:
            kv, _, nk = _counter_means(os.path.join(base, f"{cn}_{raw}"), preds[k], psteps)
            traffic.setdefault(k, {})[cn] = dict(kib=kv[cn], n=nk, bytes=kv[cn] * 1024.0 * factor)

    derived = {}
    for k in spec["kernels"]:
        q = per[k]
        sq = q["sq"]
        dur_ns = sum(q["pmc_durs"]) / len(q["pmc_durs"])
        cycles = sq["GRBM_GUI_ACTIVE"] / XCDS
        simd_cycles = CUS * SIMDS_PER_CU * cycles
        hbm_k = traffic[k]["FETCH_SIZE"]["bytes"] + traffic[k]["WRITE_SIZE"]["bytes"]
        derived[k] = {
            "kernel": q["name"],
            "duration_ms_under_counters": dur_ns * 1e-6,
            # GRBM_GUI_ACTIVE also counts the GPU's activity around a dispatch:
            # no clock figure for dispatches too short for that to vanish
            "engine_clock_ghz": cycles / dur_ns if dur_ns >= 1e5 else None,
            "mfma_busy": sq["SQ_VALU_MFMA_BUSY_CYCLES"] / simd_cycles,
            "mfma_valu_coexec": sq["SQ_VALU_MFMA_COEXEC_CYCLES"] / simd_cycles,
            "lds_busy": sq["SQ_LDS_IDX_ACTIVE"] / (CUS * cycles),
            "lds_bank_conflict_cycles": sq["SQ_LDS_BANK_CONFLICT"],
            "hbm_gbps_under_counters": hbm_k / dur_ns,
            "per_wave": {n: sq[c_] / sq["SQ_WAVES"] for n, c_ in (
                ("valu", "SQ_INSTS_VALU"), ("mfma", "SQ_INSTS_MFMA"), ("lds", "SQ_INSTS_LDS"),
                ("salu", "SQ_INSTS_SALU"), ("v_exp_f32", "SQ_INSTS_VALU_TRANS_F32"))},
            "trace_avg_ms": float(_col(q["st"], "AverageNs", "Average_Ns")) * 1e-6,
            "trace_timed_ms": sum(q["durs"]) / len(q["durs"]) * 1e-6,
            "hbm_bytes_per_launch": hbm_k,
            "waves": sq["SQ_WAVES"],
        }
    hbm = sum(derived[k]["hbm_bytes_per_launch"] for k in spec["kernels"])
    prefix = spec["prefix"]
    summary = f"profiles/{prefix}_{tag}_sq_counters.md"
    if len(spec["kernels"]) == 1:
        entry = dict(derived[spec["kernels"][0]], summary=summary)
        tentry = {"kernel": per[spec["kernels"][0]]["name"],
                  "fetch_bytes_per_launch": traffic[spec["kernels"][0]]["FETCH_SIZE"]["bytes"],
                  "write_bytes_per_launch": traffic[spec["kernels"][0]]["WRITE_SIZE"]["bytes"]}
    else:
        entry = {"kernels": derived, "summary": summary}
        tentry = {"kernels": {k: {"fetch_bytes_per_launch": traffic[k]["FETCH_SIZE"]["bytes"],
                                  "write_bytes_per_launch": traffic[k]["WRITE_SIZE"]["bytes"]}
                              for k in spec["kernels"]}}
    tentry.update(hbm_bytes_per_launch=hbm, algorithmic_bytes_per_launch=spec["algo"])
    _merge_record(os.path.join(pdir, os.path.basename(_record_path("counters", fam))), sha, wl, entry)
    _merge_record(os.path.join(pdir, os.path.basename(_record_path("traffic", fam))), sha, wl, tentry,
                  extra={"calibration": {"copy_bytes": COPY_MIB << 20, "fetch_factor": calib["FETCH_SIZE"]["factor"],
                                         "write_factor": calib["WRITE_SIZE"]["factor"]}})

    head = (f"Kernel source sha256 ({srcs}): `{sha}`\n\n"
            + "".join(f"Kernel: `{per[k]['name']}`\n\n" for k in spec["kernels"])
            + "Written by `python bench.py --collect-counters --workload " + wl + "` from the raw rocprofv3 output "
            "of the commands below ($REPO being the repository's path on the MI355X box).\n")
    md = [f"# {prefix}, {title} — kernel trace\n", head, "```", cmds["trace"], "```\n",
          "| kernel | calls | average (ns) | min (ns) | max (ns) | stddev (ns) | last timed calls (ns) | TFLOP/s there |",
          "|---|---|---|---|---|---|---|---|"]
    for k in spec["kernels"]:
        q, st = per[k], per[k]["st"]
        tms = sum(q["durs"]) / len(q["durs"])
        fl = spec["flops"].get(k)
        md.append(f"| `{k}` | {_col(st, 'Calls')} | {float(_col(st, 'AverageNs', 'Average_Ns')):.0f} | "
                  f"{_col(st, 'MinNs', 'Min_Ns')} | {_col(st, 'MaxNs', 'Max_Ns')} | "
                  f"{float(_col(st, 'StdDev', 'Stddev')):.0f} | {tms:.0f} (last {len(q['durs'])}) | "
                  + (f"{fl / tms * 1e-3:.1f}" if fl else "—") + " |")
    md += ["", f"Each kernel's calls include the {warm} warm-up steps; the last-calls column covers the bench's "
           "last timed loop" + (" (attention launches only)" if wl.startswith("fp8") else "")
           + ". The first warm-up calls run while the engine clock ramps up."]
    open(os.path.join(pdir, f"{prefix}_{tag}_kernel_trace.md"), "w").write("\n".join(md) + "\n")

    names = sorted(set().union(*(per[k]["sq"] for k in spec["kernels"])))
    md = [f"# {prefix}, {title} — SQ counters\n", head, "One counter pass per run:\n", "```", *cmds["sq"], "```\n",
          f"Mean per dispatch over each kernel's last {psteps} dispatches:\n",
          "| counter | " + " | ".join(f"`{k}`" for k in spec["kernels"]) + " |",
          "|---|" + "---|" * len(spec["kernels"])]
    md += [f"| {n} | " + " | ".join(f"{per[k]['sq'].get(n, float('nan')):.6g}" for k in spec["kernels"]) + " |"
           for n in names]
    md += ["", f"Derived (GRBM_GUI_ACTIVE is summed over the {XCDS} XCDs; {CUS} CUs x {SIMDS_PER_CU} SIMDs; each "
           "duration is the mean of the counted dispatches in the GRBM pass's kernel trace):", ""]
    for k in spec["kernels"]:
        d_ = derived[k]
        clk = (f"engine clock ≈ {d_['engine_clock_ghz']:.2f} GHz" if d_["engine_clock_ghz"] is not None
               else "too short for a clock figure")
        md += [f"- `{k}`: duration under counters {d_['duration_ms_under_counters']:.4f} ms; {clk}; "
               f"MFMA busy {d_['mfma_busy']:.3f} of SIMD cycles, MFMA and VALU "
               f"co-issue {d_['mfma_valu_coexec']:.3f}; LDS busy ≈ {d_['lds_busy']:.3f} of CU cycles, bank-conflict "
               f"cycles {d_['lds_bank_conflict_cycles']:.0f}; HBM {d_['hbm_gbps_under_counters']:.0f} GB/s; per wave: "
               + ", ".join(f"{n} {v:.0f}" for n, v in d_["per_wave"].items())]
        pw = d_["per_wave"]
        nv, nt = pw["valu"] - pw["mfma"], pw["v_exp_f32"]
        tv = d_["waves"] * ((nv - nt) * VALU_CYCLES + nt * TRANS_CYCLES) / (SIMDS * ENGINE_GHZ * 1e9) * 1e3
        md += [f"  - VALU issue bound of `{k}` ({nv:.0f} VALU instructions per wave besides MFMA, {nt:.0f} of them "
               f"transcendental; {VALU_CYCLES:g} / {TRANS_CYCLES:g} SIMD cycles per wave64 instruction, {SIMDS} SIMDs at "
               f"{ENGINE_GHZ} GHz): {tv:.4f} ms, {tv / d_['duration_ms_under_counters']:.3f} of the duration under counters"]
        # the forward's softmax phases run one wave per SIMD at a time; the
        # other kernels' waves run free, so this bound is the forward's alone
        t1 = one_wave_bound_ms(d_["waves"], nv, nt, d_["engine_clock_ghz"]) if spec["family"] == "fwd" else None
        if t1 is not None:
            md += [f"  - One-wave issue bound (the same work issued one wave per SIMD at a time, "
                   f"{ONE_WAVE_VALU_CYCLES:g} / {ONE_WAVE_TRANS_CYCLES:g} cycles per instruction, at "
                   f"{d_['engine_clock_ghz']:.2f} GHz): {t1:.4f} ms, {t1 / d_['duration_ms_under_counters']:.3f} of the "
                   "duration under counters"]
    open(os.path.join(pdir, f"{prefix}_{tag}_sq_counters.md"), "w").write("\n".join(md) + "\n")

    md = [f"# {prefix}, {title} — HBM traffic\n", head, "```", *cmds["traffic"], "```\n",
          f"Copy calibration ({COPY_MIB} MiB through `{calib['FETCH_SIZE']['copy_kernel']}`): FETCH_SIZE "
          f"{calib['FETCH_SIZE']['copy_kib']:.1f} KiB/dispatch (n={calib['FETCH_SIZE']['copy_n']}), factor "
          f"{calib['FETCH_SIZE']['factor']:.4f}; WRITE_SIZE {calib['WRITE_SIZE']['copy_kib']:.1f} KiB/dispatch "
          f"(n={calib['WRITE_SIZE']['copy_n']}), factor {calib['WRITE_SIZE']['factor']:.4f}.\n",
          "| kernel | FETCH_SIZE (KiB/dispatch) | WRITE_SIZE (KiB/dispatch) | bytes read | bytes written |",
          "|---|---|---|---|---|"]
    for k in spec["kernels"]:
        t = traffic[k]
        md.append(f"| `{k}` | {t['FETCH_SIZE']['kib']:.1f} (n={t['FETCH_SIZE']['n']}) | {t['WRITE_SIZE']['kib']:.1f} "
                  f"(n={t['WRITE_SIZE']['n']}) | {t['FETCH_SIZE']['bytes']:,.0f} | {t['WRITE_SIZE']['bytes']:,.0f} |")
    md += ["", f"Kernel counts are the mean of each kernel's last {psteps} dispatches.", "",
           f"HBM traffic per call: {hbm:,.0f} B. Algorithmic bytes ({spec['algo_what']}): {spec['algo']:,} B; "
           f"ratio {hbm / spec['algo']:.4f}."]
    open(os.path.join(pdir, f"{prefix}_{tag}_traffic.md"), "w").write("\n".join(md) + "\n")
    print(json.dumps({"counters": entry, "hbm_bytes_per_launch": hbm, "algorithmic_bytes": spec["algo"]}),
          flush=True)


if __name__ == "__main__":
    main()
