#!/usr/bin/env python3
"""Throughput of the fused exact-attention hot path on one MI355X.

One step = the whole path on one batch of synthetic input: the forward kernel
(O, LSE) followed by the two backward stages (dQ, which also forms the row sums
D, then dK/dV) of the fwd+bwd workload c5 (bf16, B=2, H=16, N=4096, d=128,
causal).  Inputs are
resident in device memory before the timed region starts.  Each kernel is
bracketed by HIP events on the stream it is launched on, so the per-kernel
averages (and the roofline of the dominant kernel) are measured live.

Prints ONE JSON line on stdout.  Everything else goes to stderr.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

Other modes (each prints its own JSON): --variants (block-sparse and dropout
against dense), --sweep (rates across shapes), --fwd-workload NAME (one forward
workload), --copy-calibration MIB, and the report writers --counters-from,
--trace-summary-from.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "attention TFLOP/s (fwd, fwd+bwd; causal-adjusted) and % of MI355X bf16 MFMA peak"
PEAK_TFLOPS = {"bf16": 2500.0, "f16": 2500.0, "f32": 157.3, "e4m3": 5000.0}   # MI355X dense matrix peaks
PEAK_HBM_GBS = 8000.0
KERNEL_SOURCES = ["exact_io_aware_51_amd/csrc/fa_fwd.hip", "exact_io_aware_51_amd/csrc/fa_fwd16.hip",
                  "exact_io_aware_51_amd/csrc/fa_fwd16_d128.hip",
                  "exact_io_aware_51_amd/csrc/fa_fwd8.hip", "exact_io_aware_51_amd/csrc/fa_decode.hip",
                  "exact_io_aware_51_amd/csrc/fa_bwd.hip", "exact_io_aware_51_amd/csrc/fa_bwd16.hip",
                  "exact_io_aware_51_amd/csrc/fa_bwd16_drop.hip", "exact_io_aware_51_amd/build.py",
                  "exact_io_aware_51_amd/csrc/fa_device.h", "exact_io_aware_51_amd/csrc/fa_tile16.h"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_models(w):
    """Algorithmic flops and bytes per launch of each kernel of one step.

    Flops count only the products the method needs (forward: S and PV; backward:
    the S recompute, dV, dP, dQ, dK), halved under the causal mask.  The dQ
    kernel also recomputes S and dP, which is extra work and not counted.
    Bytes count each input read once and each output written once.
    """
    e = 2 if w.dtype in ("bf16", "f16") else 4
    bh, n, d = w.B * w.H, w.N, w.d
    half = 0.5 if w.causal else 1.0
    nn = float(n) * n * d * bh * half
    t = float(n) * d * e * bh   # one [B,H,N,d] tensor
    r = 4.0 * n * bh            # one fp32 [B,H,N] vector
    return {
        "fwd": {"flops": 4 * nn, "bytes": 3 * t + t + r},
        # dQ, first backward stage: reads q, k, v, o, dout and lse, writes dq and the row sums D
        "bwd_dq": {"flops": 2 * nn, "bytes": 5 * t + r + t + r},
        # dK/dV: reads q, k, v, dout, lse and D, writes dk and dv
        "bwd_dkdv": {"flops": 8 * nn, "bytes": 4 * t + 2 * r + 2 * t},
    }


def source_digest():
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_for(kernel):
    """HBM bytes per launch from committed counter runs, or None if absent or stale."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    entry = t.get("kernels", {}).get(kernel)
    if not entry or t.get("source_digest") != source_digest():
        return None
    return entry.get("hbm_bytes_per_launch")


STEP_KERNELS = {"fwd16_kernel": "fwd", "dkdv": "bwd_dkdv", "dq16_kernel": "bwd_dq"}  # dkdv16_kernel, dkdv16n_kernel, dkdv32s_kernel


# --------------------------------------------------------------- counter reports
N_XCD, N_CU, MFMA_FLOP_PER_CU_CLK = 8, 256, 4096   # MI355X: 2.5 PFLOP/s dense bf16 = 256 CU x 2.4 GHz x 4096
COUNTER_PASSES = [
    "SQ_VALU_MFMA_BUSY_CYCLES SQ_VALU_MFMA_COEXEC_CYCLES SQ_INSTS_VALU SQ_ACTIVE_INST_VALU SQ_INSTS_MFMA "
    "SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_INSTS_VALU_MFMA_MOPS_F16 SQ_WAVES GRBM_GUI_ACTIVE",
    "SQ_LDS_BANK_CONFLICT SQ_ACTIVE_INST_LDS SQ_INSTS_LDS SQ_WAIT_INST_LDS SQ_WAIT_INST_ANY SQ_INSTS_VALU_TRANS_F32 "
    "SQ_BUSY_CU_CYCLES SQ_INSTS_SALU GRBM_GUI_ACTIVE",
    "FETCH_SIZE",
    "WRITE_SIZE",
]
WORKLOAD_CMDS = {  # the command each counter report profiles (from the repository root)
    "c5": "python3 bench.py --steps 5 --warmup 2 --no-cpu-baseline --no-fwd-workloads",
    "c3": "python3 bench.py --fwd-workload c3 --steps 5 --warmup 2",
    "c4": "python3 bench.py --fwd-workload c4 --steps 5 --warmup 2",
}
FWD_KERNELS = {"fwd16_kernel": "fwd", "fwd_kernel": "fwd"}


def _pmc_per_kernel(run_dir):
    """{kernel: {counter: mean per dispatch}} and {kernel: dispatches} from a --pmc run directory."""
    import csv
    import glob
    files = glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no *counter_collection.csv under {run_dir}")
    per = {}
    for fn in files:
        with open(fn, newline="") as f:
            for row in csv.DictReader(f):
                key = (row["Kernel_Name"], row["Dispatch_Id"], row["Counter_Name"])
                per[key] = per.get(key, 0.0) + float(row["Counter_Value"])
    acc, disp = {}, {}
    for (kname, did, cname), v in per.items():
        acc.setdefault(kname, {}).setdefault(cname, []).append(v)
        disp.setdefault(kname, set()).add(did)
    return ({k: {c: sum(v) / len(v) for c, v in cs.items()} for k, cs in acc.items()},
            {k: len(v) for k, v in disp.items()})


def _trace_stats(run_dir):
    """{kernel: (calls, average ns, min ns)} from a --kernel-trace --stats run directory."""
    import csv
    import glob
    files = glob.glob(os.path.join(run_dir, "**", "*kernel_stats.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no *kernel_stats.csv under {run_dir}")
    out = {}
    with open(files[0], newline="") as f:
        for row in csv.DictReader(f):
            out[row["Name"]] = (int(row["Calls"]), float(row["AverageNs"]), float(row["MinNs"]))
    return out


def _stage_of(kname, w):
    if w.mode == "fwd+bwd":
        return next((v for k, v in STEP_KERNELS.items() if k in kname), None)
    return next((v for k, v in FWD_KERNELS.items() if k in kname), None)


def write_counter_report(prof_dir, w, cal_dir):
    """profiles/<workload>_counters.{json,md} from rocprofv3 runs under prof_dir:
    trace/ (--kernel-trace --stats) and pmc1 .. pmc4 (the COUNTER_PASSES of
    WORKLOAD_CMDS[w.name]); cal_dir holds copy_FETCH_SIZE / copy_WRITE_SIZE
    (bench.py --copy-calibration 1024) for the byte counters' scale."""
    copy_bytes = 1024 << 20
    cf, _ = _pmc_per_kernel(os.path.join(cal_dir, "copy_FETCH_SIZE"))
    cw, _ = _pmc_per_kernel(os.path.join(cal_dir, "copy_WRITE_SIZE"))
    cname = next(k for k in cf if "copyBuffer" in k)
    ff = copy_bytes / (cf[cname]["FETCH_SIZE"] * 1024.0)
    wf = copy_bytes / (cw[cname]["WRITE_SIZE"] * 1024.0)
    trace = _trace_stats(os.path.join(prof_dir, "trace"))
    ctr, calls = {}, {}
    for i in range(1, len(COUNTER_PASSES) + 1):
        c, n = _pmc_per_kernel(os.path.join(prof_dir, f"pmc{i}"))
        for k, v in c.items():
            ctr.setdefault(k, {}).update(v)
            calls[k] = max(calls.get(k, 0), n[k])
    models = kernel_models(w) if w.mode == "fwd+bwd" else {"fwd": kernel_models(w)["fwd"]}
    e = 2 if w.dtype in ("bf16", "f16") else 4
    bh, n_, d_ = w.B * w.H, w.N, w.d
    naive_fwd = bh * (4.0 * n_ * n_ * e + 4.0 * n_ * d_ * e)  # write S, read S, write P, read P; Q, K, V, O once
    rows = {}
    for kname, c in ctr.items():
        stage = _stage_of(kname, w)
        if stage is None or stage not in models:
            continue
        m = models[stage]
        tr = next((v for k, v in trace.items() if k == kname), None)
        avg_ns = tr[1] if tr else None
        gui = c.get("GRBM_GUI_ACTIVE", 0.0) / N_XCD          # cycles per XCD while the kernel ran
        simd_cycles = gui * N_CU * 4
        mops = c.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0) + c.get("SQ_INSTS_VALU_MFMA_MOPS_F16", 0.0)
        mfma_flops = 512.0 * mops
        waves = c.get("SQ_WAVES", 0.0) or 1.0
        hbm = c.get("FETCH_SIZE", 0.0) * 1024 * ff + c.get("WRITE_SIZE", 0.0) * 1024 * wf
        r = {"kernel_symbol": kname, "dispatches_counted": calls[kname],
             "trace_avg_us": round(avg_ns / 1e3, 2) if avg_ns else None,
             "clock_mhz": round(gui / (avg_ns * 1e-9) / 1e6, 1) if avg_ns and gui else None,
             "algorithmic_flops": m["flops"], "mfma_flops_executed": mfma_flops,
             "mfma_flops_over_algorithmic": round(mfma_flops / m["flops"], 3) if m["flops"] else None,
             "algorithmic_tflops_by_trace": round(m["flops"] / (avg_ns * 1e-9) / 1e12, 1) if avg_ns else None,
             "frac_of_2p5_pflops_by_trace": round(m["flops"] / (avg_ns * 1e-9) / 2.5e15, 4) if avg_ns else None,
             "mfma_util_at_measured_clock": round(mfma_flops / (MFMA_FLOP_PER_CU_CLK * N_CU * gui), 4) if gui else None,
             "mfma_busy_per_simd": round(c.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / simd_cycles, 4) if gui else None,
             "mfma_valu_coexec_per_simd": round(c.get("SQ_VALU_MFMA_COEXEC_CYCLES", 0.0) / simd_cycles, 4) if gui else None,
             "valu_active_per_simd": round(c.get("SQ_ACTIVE_INST_VALU", 0.0) / simd_cycles, 4) if gui else None,
             "valu_insts_per_wave": round(c.get("SQ_INSTS_VALU", 0.0) / waves, 1),
             "mfma_insts_per_wave": round(c.get("SQ_INSTS_MFMA", 0.0) / waves, 1),
             "exp_insts_per_wave": round(c.get("SQ_INSTS_VALU_TRANS_F32", 0.0) / waves, 1),
             "lds_insts_per_wave": round(c.get("SQ_INSTS_LDS", 0.0) / waves, 1),
             "lds_bank_conflict_cycles": c.get("SQ_LDS_BANK_CONFLICT"),
             "lds_bank_conflicts_per_lds_active_cycle": (round(c["SQ_LDS_BANK_CONFLICT"] / c["SQ_ACTIVE_INST_LDS"], 4)
                                                         if c.get("SQ_ACTIVE_INST_LDS") else None),
             "wait_lds_over_wait_any": (round(c.get("SQ_WAIT_INST_LDS", 0.0) / c["SQ_WAIT_INST_ANY"], 4)
                                        if c.get("SQ_WAIT_INST_ANY") else None),
             "waves": waves,
             "hbm_bytes": int(hbm), "algorithmic_bytes": m["bytes"],
             "hbm_over_algorithmic": round(hbm / m["bytes"], 3),
             "hbm_gbs_by_trace": round(hbm / (avg_ns * 1e-9) / 1e9, 1) if avg_ns else None,
             "raw_counters_per_dispatch": {k: round(v, 1) for k, v in sorted(c.items())}}
        if stage == "fwd":
            outs = bh * n_ * d_
            r["bytes_per_output_element"] = round(hbm / outs, 2)
            r["naive_4pass_bytes"] = naive_fwd
            r["naive_bytes_per_output_element"] = round(naive_fwd / outs, 1)
            r["naive_over_measured"] = round(naive_fwd / hbm, 1) if hbm else None
        rows[stage] = r
    cmd = WORKLOAD_CMDS[w.name]
    rep = {"workload": f"{w.name}: {w.dtype} B={w.B} H={w.H} N={w.N} d={w.d} "
                       f"{'causal' if w.causal else 'non-causal'} ({w.mode})",
           "source_digest": source_digest(),
           "commands": [f"rocprofv3 --kernel-trace --stats --output-format csv -d DIR/trace -o run -- {cmd}"] +
                       [f"timeout -s KILL 90 rocprofv3 --pmc {p} --output-format csv -d DIR/pmc{i + 1} -o run -- {cmd}"
                        for i, p in enumerate(COUNTER_PASSES)] +
                       [f"timeout -s KILL 90 rocprofv3 --pmc {c} --output-format csv -d CAL/copy_{c} -o run -- "
                        f"python3 bench.py --copy-calibration 1024" for c in ("FETCH_SIZE", "WRITE_SIZE")],
           "calibration": {"copy_kernel": cname, "fetch_factor": round(ff, 4), "write_factor": round(wf, 4)},
           "kernels": rows}
    base = os.path.join(ROOT, "profiles", f"{w.name}_counters")
    with open(base + ".json", "w") as f:
        json.dump(rep, f, indent=1)
        f.write("\n")
    with open(base + ".md", "w") as f:
        f.write(_counter_markdown(rep))
    log(f"wrote {base}.json / .md")
    if w.mode == "fwd+bwd":
        # the HBM bytes the bench line reports as roofline.traffic, tied to these sources
        t = {"source_digest": rep["source_digest"], "workload": rep["workload"],
             "from": f"profiles/{w.name}_counters.json (FETCH_SIZE and WRITE_SIZE passes, copy-calibrated)",
             "calibration": rep["calibration"],
             "kernels": {st: {"kernel_symbol": r["kernel_symbol"],
                              "fetch_kib_per_dispatch": r["raw_counters_per_dispatch"].get("FETCH_SIZE"),
                              "write_kib_per_dispatch": r["raw_counters_per_dispatch"].get("WRITE_SIZE"),
                              "hbm_bytes_per_launch": r["hbm_bytes"],
                              "algorithmic_bytes_per_launch": r["algorithmic_bytes"]} for st, r in rows.items()}}
        with open(TRAFFIC_FILE, "w") as f:
            json.dump(t, f, indent=1)
            f.write("\n")
        log(f"wrote {TRAFFIC_FILE}")
    return rep


STEP_LABELS = {"fwd": "fa_fwd", "bwd_dq": "fa_bwd_dq_rowsum", "bwd_dkdv": "fa_bwd_dkdv"}


def write_trace_summary(trace_dir, w, warmup, steps, bench_log=None, out_dir=None):
    """profiles/<workload>_step_kernel_stats.md from a rocprofv3 --kernel-trace --stats run of
    `bench.py --steps STEPS --warmup WARMUP --no-cpu-baseline`: the step is timed first, so the
    first WARMUP + STEPS dispatches of each step kernel are the step's, the last STEPS of them timed."""
    import csv
    import glob
    files = glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no *kernel_trace.csv under {trace_dir}")
    rows = list(csv.DictReader(open(files[0], newline="")))
    rows.sort(key=lambda r: int(r["Dispatch_Id"]))
    by = {}
    for r in rows:
        by.setdefault(r["Kernel_Name"], []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    # per stage, the matching kernel dispatched first is the step's (other workloads' kernels come later)
    step_kernel = {}
    for r in rows:
        stage = next((v for k, v in STEP_KERNELS.items() if k in r["Kernel_Name"]), None)
        if stage is not None and stage not in step_kernel:
            step_kernel[stage] = r["Kernel_Name"]
    models = kernel_models(w)
    n = warmup + steps
    lines, total = [], 0.0
    for stage, kname in step_kernel.items():
        durs = by[kname]
        if len(durs) < n:
            raise SystemExit(f"{kname}: {len(durs)} dispatches, fewer than warmup + steps = {n}")
        timed = durs[warmup:n]
        avg = sum(timed) / steps
        total += avg
        lines.append((stage, kname, avg, min(timed), max(timed), models[stage]["flops"] / (avg * 1e-6) / 1e12))
    lines.sort(key=lambda x: -x[2])
    events = {}
    if bench_log:  # the JSON line the profiled bench.py printed: its HIP-event figures for the same dispatches
        with open(bench_log) as f:
            line = next(x for x in f if x.startswith("{"))
        events = {k: v["ms"] * 1e3 for k, v in json.loads(line)["kernels"].items()}
    cmd = f"python3 bench.py --steps {steps} --warmup {warmup} --no-cpu-baseline"
    L = [f"# Kernel trace of the bench step: workload {w.name}, {w.dtype} B={w.B} H={w.H} N={w.N} d={w.d} "
         f"{'causal' if w.causal else 'non-causal'}", "",
         "Commands (from the repository root on the MI355X box, `cd /tmp && export TMPDIR=/tmp` first; DIR is an "
         "output folder):", "", "```",
         f"rocprofv3 --kernel-trace --stats --output-format csv -d DIR -o run -- {cmd} > LOG",
         f"python3 bench.py --trace-summary-from DIR --bench-log LOG --steps {steps} --warmup {warmup}"
         "   # writes this file",
         "```", "",
         f"bench.py times the step first ({warmup} warm-up + {steps} timed steps), so the first {n} dispatches of "
         f"each step kernel are the step's; the table averages the {steps} timed ones. Algorithmic TFLOP/s "
         "(causal-adjusted flops per launch over the traced duration) is what bench.py's roofline reports for the "
         "slowest kernel from HIP events; the last column is bench.py's own HIP-event timing of the same dispatches "
         "in this profiled run. The profiler slows the kernels: an unprofiled run of the same command is faster.",
         "",
         f"Source digest of the kernels traced: `{source_digest()}`.", "",
         "| stage | kernel | avg us | min us | max us | share of step | algorithmic TFLOP/s | of 2.5 PF "
         "| HIP events, same run (us) |",
         "|---|---|---|---|---|---|---|---|---|"]
    for stage, kname, avg, mn, mx, tf in lines:
        ev = f"{events[stage]:.1f}" if stage in events else ""
        L.append(f"| {STEP_LABELS[stage]} | `{kname}` | {avg:.1f} | {mn:.1f} | {mx:.1f} | {100 * avg / total:.1f}% | "
                 f"{tf:.1f} | {tf / PEAK_TFLOPS[w.dtype]:.4f} | {ev} |")
    L += ["", f"Step (sum of the kernels' averages): {total:.1f} us; "
              f"{sum(m['flops'] for m in models.values()) / (total * 1e-6) / 1e12:.1f} TFLOP/s over kernel time.", ""]
    sfiles = glob.glob(os.path.join(trace_dir, "**", "*kernel_stats.csv"), recursive=True)
    if sfiles:
        L += ["All dispatches of this library's kernels in the run (rocprofv3 `--stats`), including the forward-only "
              "lines of the other workloads that bench.py times after the step:", "",
              "| kernel | calls | average us | min us | max us |", "|---|---|---|---|---|"]
        for r in csv.DictReader(open(sfiles[0], newline="")):
            if "fa::" in r["Name"] or "_ZN2fa" in r["Name"]:
                L.append(f"| `{r['Name']}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                         f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} |")
        L.append("")
    out = os.path.join(out_dir or os.path.join(ROOT, "profiles"), f"{w.name}_step_kernel_stats.md")
    with open(out, "w") as f:
        f.write("\n".join(L))
    log(f"wrote {out}")


def _counter_markdown(rep):
    L = [f"# Counters: workload {rep['workload']}", "",
         "Commands (from the repository root on the MI355X box, `cd /tmp && export TMPDIR=/tmp` first; DIR and "
         "CAL are output folders):", "", "```"] + rep["commands"] + ["```", "",
         f"Byte counters scaled by a 1 GiB device copy: FETCH_SIZE x {rep['calibration']['fetch_factor']}, "
         f"WRITE_SIZE x {rep['calibration']['write_factor']}. `GRBM_GUI_ACTIVE` is summed over the 8 XCDs, so the "
         "clock is its per-XCD value over the traced kernel time. MFMA utilisation counts "
         "`SQ_INSTS_VALU_MFMA_MOPS_*` x 512 flops against 4096 flops per CU per clock at that clock; busy, "
         "co-execution and VALU-active fractions are per SIMD (1024 SIMDs).", "",
         f"Source digest of the kernels measured: `{rep['source_digest']}`.", ""]
    keys = [("trace_avg_us", "trace avg (us)"), ("clock_mhz", "clock (MHz)"),
            ("algorithmic_tflops_by_trace", "algorithmic TFLOP/s"), ("frac_of_2p5_pflops_by_trace", "of 2.5 PF"),
            ("mfma_flops_over_algorithmic", "MFMA flops / algorithmic"),
            ("mfma_util_at_measured_clock", "MFMA util at clock"), ("mfma_busy_per_simd", "MFMA busy / SIMD"),
            ("mfma_valu_coexec_per_simd", "MFMA+VALU co-exec / SIMD"), ("valu_active_per_simd", "VALU active / SIMD"),
            ("valu_insts_per_wave", "VALU insts / wave"), ("exp_insts_per_wave", "exp insts / wave"),
            ("mfma_insts_per_wave", "MFMA insts / wave"), ("lds_insts_per_wave", "LDS insts / wave"),
            ("lds_bank_conflicts_per_lds_active_cycle", "LDS bank conflict / LDS active"),
            ("wait_lds_over_wait_any", "LDS wait / any wait"),
            ("hbm_over_algorithmic", "HBM bytes / algorithmic"), ("hbm_gbs_by_trace", "HBM GB/s"),
            ("bytes_per_output_element", "HBM bytes per output element"),
            ("naive_bytes_per_output_element", "naive 4-pass bytes per output element"),
            ("naive_over_measured", "naive / measured bytes")]
    stages = list(rep["kernels"])
    L.append("| metric | " + " | ".join(stages) + " |")
    L.append("|---|" + "---|" * len(stages))
    for k, label in keys:
        vals = [rep["kernels"][s].get(k) for s in stages]
        if all(v is None for v in vals):
            continue
        L.append(f"| {label} | " + " | ".join("" if v is None else str(v) for v in vals) + " |")
    L.append("")
    L.append("Kernel symbols: " + "; ".join(f"{s}: `{rep['kernels'][s]['kernel_symbol']}`" for s in stages))
    L.append("")
    return "\n".join(L)


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline(w, seconds):
    """The fp64 oracle on whole heads of the same workload, one (batch, head) per
    host thread (one BLAS thread each), until `seconds` have passed.

    Threads: the cores this process may run on (os.sched_getaffinity), at most
    16, a GPU machine's CPU share per GPU.  numpy releases the interpreter lock in
    its array loops and BLAS calls, so the heads run in parallel."""
    import concurrent.futures

    from threadpoolctl import threadpool_info, threadpool_limits

    import oracle
    from exact_io_aware_51_amd import workloads as W
    q, k, v, do = W.make_inputs(w)
    models = kernel_models(w)
    per_head = sum(m["flops"] for m in models.values()) / (w.B * w.H)
    heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    host = len(os.sched_getaffinity(0))
    workers = max(1, min(16, host))
    blas = [f"{p.get('internal_api')} {p.get('version')}" for p in threadpool_info() if p.get("user_api") == "blas"]

    def one(bh):
        b, h = bh
        sl = slice(b, b + 1), slice(h, h + 1)
        oracle.attention_forward(q[sl], k[sl], v[sl], w.scale, w.causal)
        oracle.attention_backward(q[sl], k[sl], v[sl], do[sl], w.scale, w.causal)

    done, t_end = 0, None
    with threadpool_limits(limits=1, user_api="blas"):
        with concurrent.futures.ThreadPoolExecutor(max_workers=workers) as ex:
            t0 = time.perf_counter()
            todo = iter(heads)
            running = {ex.submit(one, bh) for bh in [next(todo) for _ in range(min(workers, len(heads)))]}
            while running:
                fin, running = concurrent.futures.wait(running, return_when=concurrent.futures.FIRST_COMPLETED)
                for f in fin:
                    f.result()
                    done += 1
                t_end = time.perf_counter()
                if t_end - t0 < seconds:
                    for _ in fin:
                        nxt = next(todo, None)
                        if nxt is not None:
                            running.add(ex.submit(one, nxt))
    dt = t_end - t0
    return {"value": per_head * done / dt / 1e12, "unit": "TFLOP/s", "cores": workers, "kind": "oracle",
            "sample": f"{done} of {len(heads)} heads of workload {w.name} (fwd+bwd per head, fp64 numpy, one head "
                      f"per thread, {dt:.1f} s; algorithmic causal-adjusted flops)",
            "host_cores": host, "cpu_model": _cpu_model(), "blas": ", ".join(blas) or "unknown",
            "blas_threads_per_worker": 1}


class Runner:
    """Device buffers and raw C-ABI calls for one workload."""

    def __init__(self, w, dev):
        import torch

        import exact_io_aware_51_amd as fa
        from exact_io_aware_51_amd import workloads as W
        self.fa, self.w = fa, w
        with_grad = w.mode == "fwd+bwd"
        ins = [t.to(dev) for t in W.make_inputs(w, with_grad=with_grad)]
        self.q, self.k, self.v = ins[:3]
        self.do = ins[3] if with_grad else None
        self.o = torch.empty_like(self.q)
        self.lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)
        self.code = {"f32": fa.FA_F32, "f16": fa.FA_F16, "bf16": fa.FA_BF16}[w.dtype]
        if with_grad:
            self.dq, self.dk, self.dv = (torch.empty_like(self.q) for _ in range(3))
            self.wsb = fa.fa_bwd_workspace_bytes(w.B, w.H, w.N, w.d, self.code)
            self.ws = torch.empty(self.wsb, dtype=torch.uint8, device=dev)
        self.stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
        self.dims = (w.B, w.H, w.N, w.d)

    def _ok(self, st, what):
        if st != 0:
            raise RuntimeError(f"{what}: {self.fa.fa_status_string(st)}")

    def fwd(self):
        w = self.w
        self._ok(self.fa.fa_fwd(self.q.data_ptr(), self.k.data_ptr(), self.v.data_ptr(), self.o.data_ptr(),
                                self.lse.data_ptr(), *self.dims, w.scale, int(w.causal), self.code, self.stream),
                 "fa_fwd")

    def dq_rowsum(self):
        w = self.w
        self._ok(self.fa.fa_bwd_dq_rowsum(self.q.data_ptr(), self.k.data_ptr(), self.v.data_ptr(),
                                          self.o.data_ptr(), self.do.data_ptr(), self.lse.data_ptr(),
                                          self.ws.data_ptr(), self.wsb, self.dq.data_ptr(), *self.dims, w.scale,
                                          int(w.causal), self.code, self.stream), "fa_bwd_dq_rowsum")

    def dkdv(self):
        w = self.w
        self._ok(self.fa.fa_bwd_dkdv(self.q.data_ptr(), self.k.data_ptr(), self.v.data_ptr(), self.do.data_ptr(),
                                     self.lse.data_ptr(), self.ws.data_ptr(), self.wsb, self.dk.data_ptr(),
                                     self.dv.data_ptr(), *self.dims, w.scale, int(w.causal), self.code,
                                     self.stream), "fa_bwd_dkdv")



def _spread(times_ms):
    """Median and minimum of per-launch times (ms)."""
    t = sorted(times_ms)
    n = len(t)
    med = t[n // 2] if n % 2 else 0.5 * (t[n // 2 - 1] + t[n // 2])
    return {"ms_median": round(med, 4), "ms_min": round(t[0], 4)}


def time_fwd_only(name, dev, iters=20, warmup=3):
    import torch

    from exact_io_aware_51_amd import workloads as W
    w = W.WORKLOADS[name]
    r = Runner(w, dev)
    for _ in range(warmup):
        r.fwd()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * iters)]
    torch.cuda.synchronize()
    for i in range(iters):
        ev[2 * i].record()
        r.fwd()
        ev[2 * i + 1].record()
    torch.cuda.synchronize()
    times = [ev[2 * i].elapsed_time(ev[2 * i + 1]) for i in range(iters)]
    ms = sum(times) / iters
    tf = w.fwd_flops() / (ms * 1e-3) / 1e12
    return {"ms": round(ms, 4), **_spread(times), "tflops": round(tf, 1),
            "frac_of_peak": round(tf / PEAK_TFLOPS[w.dtype], 4),
            "shape": f"{w.dtype} B={w.B} H={w.H} N={w.N} d={w.d} {'causal' if w.causal else 'non-causal'}"}


def _amd_smi(args):
    """Parsed JSON of `amd-smi <args> --json`, or None if the tool or its output is unavailable."""
    import subprocess
    try:
        r = subprocess.run(["amd-smi", *args, "--json"], capture_output=True, text=True, timeout=15)
        return json.loads(r.stdout)
    except Exception:  # noqa: BLE001 - best effort: a missing tool only drops the field
        return None


def _walk(x, visit):
    if isinstance(x, dict):
        for key, val in x.items():
            if not visit(key, val):
                _walk(val, visit)
    elif isinstance(x, list):
        for val in x:
            _walk(val, visit)


def _gfx_clocks_mhz():
    """Current GFX clock of every XCD from amd-smi (MHz), or [] if it cannot be read."""
    out = []

    def visit(key, val):
        if key.startswith("gfx_") and isinstance(val, dict) and isinstance(val.get("clk"), dict):
            v = val["clk"].get("value")
            if isinstance(v, (int, float)):
                out.append(float(v))
            return True
        return False
    _walk(_amd_smi(["metric", "--clock"]), visit)
    return out


def _socket_power_w():
    """Current socket power of the GPU from amd-smi (W), or None if it cannot be read."""
    out = []

    def visit(key, val):
        if key == "socket_power" and isinstance(val, dict) and isinstance(val.get("value"), (int, float)):
            out.append(float(val["value"]))
            return True
        return False
    _walk(_amd_smi(["metric", "--power"]), visit)
    return out[0] if out else None


def sample_under_load(run, seconds=3.0):
    """Mean GFX clock (MHz) and median socket power (W), sampled with amd-smi while run() is called
    back to back for about `seconds`; None if amd-smi gives no clock."""
    import threading

    import torch
    clocks, powers, stop = [], [], threading.Event()

    def sampler():
        while not stop.is_set():
            c = _gfx_clocks_mhz()
            if not c:
                return
            clocks.append(sum(c) / len(c))
            pw = _socket_power_w()
            if pw is not None:
                powers.append(pw)
    run()
    torch.cuda.synchronize()
    th = threading.Thread(target=sampler, daemon=True)
    th.start()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        run()
        torch.cuda.synchronize()
    stop.set()
    th.join(timeout=30)
    if len(clocks) < 2:
        return None
    busy = clocks[1:]  # the first sample may predate the load
    pw = sorted(powers[1:])
    return {"gfx_mhz_mean": round(sum(busy) / len(busy), 1), "socket_power_w": pw[len(pw) // 2] if pw else None,
            "samples": len(busy), "source": "amd-smi metric --clock / --power"}


def clock_under_load(name, dev, seconds=3.0):
    """GFX clock and socket power while workload `name`'s forward runs back to back."""
    from exact_io_aware_51_amd import workloads as W
    r = Runner(W.WORKLOADS[name], dev)
    got = sample_under_load(r.fwd, seconds)
    if got is None:
        return None
    return {"workload": f"{name} forward", **got}


def matmul_ceiling(dev, n=8192, iters=10, seconds=3.0):
    """Context, not part of the path: the dense bf16 matrix rate a vendor GEMM (torch.matmul, which
    calls hipBLASLt) reaches on this GPU, n x n x n, with the clock and power it runs at.  It shows
    what the matrix cores deliver under the board's power limit, next to the 2.5 PFLOP/s peak that
    assumes the 2.4 GHz clock."""
    import torch
    g = torch.Generator(device=dev).manual_seed(0)
    a = torch.randn(n, n, device=dev, dtype=torch.bfloat16, generator=g)
    b = torch.randn(n, n, device=dev, dtype=torch.bfloat16, generator=g)
    c = torch.empty(n, n, device=dev, dtype=torch.bfloat16)

    def run():
        for _ in range(iters):
            torch.matmul(a, b, out=c)
    run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    run()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / iters
    tf = 2.0 * n ** 3 / (ms * 1e-3) / 1e12
    out = {"what": f"torch.matmul bf16 {n}x{n}x{n} (hipBLASLt), context only", "ms": round(ms, 4),
           "tflops": round(tf, 1), "frac_of_peak": round(tf / PEAK_TFLOPS["bf16"], 4)}
    load = sample_under_load(run, seconds)
    if load is not None:
        out.update({k: load[k] for k in ("gfx_mhz_mean", "socket_power_w")})
    return out


def time_fwd_fp8(name, dev, iters=20, warmup=3, fmt="e4m3"):
    """The forward of workload `name`'s shape on 8-bit inputs of format `fmt` (fa_fwd_fp8_fmt), against the
    8-bit matrix peak."""
    import math

    import torch

    import exact_io_aware_51_amd as fa
    from exact_io_aware_51_amd import workloads as W
    w = W.WORKLOADS[name]
    q8, k8, v8, ds = W.fp8_inputs(w.B, w.H, w.N, w.d, w.seed, q_scale=w.q_scale, v_uniform=w.v_uniform, fmt=fmt)
    code = {"e4m3": fa.FA_FP8_E4M3, "e5m2": fa.FA_FP8_E5M2}[fmt]
    q8, k8, v8 = q8.to(dev), k8.to(dev), v8.to(dev)
    o = torch.empty((w.B, w.H, w.N, w.d), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)

    def run():
        st = fa.fa_fwd_fp8_fmt(q8.data_ptr(), k8.data_ptr(), v8.data_ptr(), o.data_ptr(), lse.data_ptr(), w.B,
                               w.H, w.N, w.d, w.scale, int(w.causal), ds[0], ds[1], ds[2], code, stream)
        if st != 0:
            raise RuntimeError(f"fa_fwd_fp8_fmt: {fa.fa_status_string(st)}")
    for _ in range(warmup):
        run()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * iters)]
    torch.cuda.synchronize()
    for i in range(iters):
        ev[2 * i].record()
        run()
        ev[2 * i + 1].record()
    torch.cuda.synchronize()
    times = [ev[2 * i].elapsed_time(ev[2 * i + 1]) for i in range(iters)]
    ms = sum(times) / iters
    tf = w.fwd_flops() / (ms * 1e-3) / 1e12
    assert math.isfinite(float(o.float().abs().max()))
    return {"ms": round(ms, 4), **_spread(times), "tflops": round(tf, 1),
            "frac_of_peak": round(tf / PEAK_TFLOPS["e4m3"], 4),
            "shape": f"{fmt} in, bf16 out, B={w.B} H={w.H} N={w.N} d={w.d} {'causal' if w.causal else 'non-causal'}"}


def time_variants(dev, iters=10, warmup=2):
    """Block-sparse and dropout entry points against the dense ones on the same inputs
    (bf16): forward and whole backward, time per call and the ratio to dense."""
    import torch

    import exact_io_aware_51_amd as fa
    from exact_io_aware_51_amd import workloads as W

    def timed(fn):
        for _ in range(warmup):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(iters):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / iters

    out = {"sparse": {}, "dropout": {}}
    for B, H, N, d in ((1, 8, 32768, 128), (2, 16, 4096, 128)):
        q, k, v, do = (t.to(dev) for t in W.kv_inputs(B, H, N, N, d, "bf16", 4242))
        o, lse = fa.forward(q, k, v, causal=True)
        fd = timed(lambda: fa.forward(q, k, v, causal=True))
        bd = timed(lambda: fa.backward(q, k, v, o, lse, do, causal=True))
        for keep in (1.0, 0.5, 0.25):
            m = W.block_mask(B, H, N, keep, 77).to(dev)
            if keep == 1.0:
                m.fill_(1)
            os_, ls_ = fa.forward_sparse(q, k, v, m, causal=True)
            fs = timed(lambda: fa.forward_sparse(q, k, v, m, causal=True))
            bs = timed(lambda: fa.backward_sparse(q, k, v, os_, ls_, do, m, causal=True))
            out["sparse"][f"B={B} H={H} N={N} d={d} causal, {int(keep * 100)}% kept"] = {
                "fwd_ms": round(fs, 4), "fwd_vs_dense": round(fs / fd, 3),
                "bwd_ms": round(bs, 4), "bwd_vs_dense": round(bs / bd, 3)}
    for B, H, N, d, causal in ((1, 16, 16384, 128, False), (1, 16, 16384, 128, True), (2, 16, 4096, 128, True),
                               (4, 16, 4096, 64, True)):
        q, k, v, do = (t.to(dev) for t in W.kv_inputs(B, H, N, N, d, "bf16", 4343))
        o, lse = fa.forward(q, k, v, causal=causal)
        fd = timed(lambda: fa.forward(q, k, v, causal=causal))
        bd = timed(lambda: fa.backward(q, k, v, o, lse, do, causal=causal))
        od, ld = fa.forward_dropout(q, k, v, 0.1, 1234, causal=causal)
        fr = timed(lambda: fa.forward_dropout(q, k, v, 0.1, 1234, causal=causal))
        br = timed(lambda: fa.backward_dropout(q, k, v, od, ld, do, 0.1, 1234, causal=causal))
        out["dropout"][f"B={B} H={H} N={N} d={d} {'causal' if causal else 'non-causal'}, p=0.1"] = {
            "fwd_ms": round(fr, 4), "fwd_vs_dense": round(fr / fd, 3),
            "bwd_ms": round(br, 4), "bwd_vs_dense": round(br / bd, 3)}
    return out


SWEEP_SHAPES = ((8, 16, 1024), (4, 16, 2048), (2, 16, 4096), (1, 16, 8192), (1, 16, 16384), (1, 8, 32768))


def time_sweep(dev, rounds=5):
    """Forward, dQ (with the row sums) and dK/dV across sequence lengths, head sizes and masks
    (bf16, seeded N(0,1) inputs): best of `rounds` timed loops per kernel, TFLOP/s with causal
    flops halved; the backward's rate is its algorithmic 10 N_eff d over the two kernels' times."""
    import torch

    from exact_io_aware_51_amd import workloads as W

    def best(fn, iters):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        t = float("inf")
        for _ in range(rounds):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(iters):
                fn()
            e1.record()
            torch.cuda.synchronize()
            t = min(t, e0.elapsed_time(e1) / iters)
        return t

    rows = []
    for B, H, N in SWEEP_SHAPES:
        for d in (64, 128):
            for causal in (True, False):
                w = W.shape_case(B, H, N, d, "bf16", causal, seed=5)
                r = Runner(w, dev)
                nn = B * H * N * N * d * (0.5 if causal else 1.0)
                iters = max(2, int(3e11 / (14 * nn)) + 1)
                r.fwd()
                r.dq_rowsum()
                tf, tq, tk = best(r.fwd, iters), best(r.dq_rowsum, iters), best(r.dkdv, iters)
                rows.append({"B": B, "H": H, "N": N, "d": d, "causal": causal,
                             "fwd_tflops": round(4 * nn / tf / 1e9, 1), "bwd_tflops": round(10 * nn / (tq + tk) / 1e9, 1),
                             "fwd_ms": round(tf, 4), "dq_ms": round(tq, 4), "dkdv_ms": round(tk, 4)})
                log(f"bench: sweep B={B} H={H} N={N} d={d} causal={causal}")
                del r
                torch.cuda.empty_cache()
    return rows


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="c5", help="fwd+bwd workload timed as the step")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-fwd-workloads", action="store_true", help="skip the forward-only lines for c1..c4")
    ap.add_argument("--sweep", action="store_true",
                    help="time the forward, dQ and dK/dV across sequence lengths, head sizes and masks (JSON)")
    ap.add_argument("--variants", action="store_true",
                    help="diagnostic: block-sparse and dropout entry points against dense, one JSON line")
    ap.add_argument("--fwd-workload", default=None,
                    help="diagnostic: time only the forward kernel of this workload (c1..c5), one JSON line")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="diagnostic: run a plain device copy of MIB MiB five times (counter calibration)")
    ap.add_argument("--trace-summary-from", default=None, metavar="DIR",
                    help="write profiles/<workload>_step_kernel_stats.md from a rocprofv3 --kernel-trace --stats run "
                         "of bench.py --steps S --warmup W --no-cpu-baseline under DIR (pass the same S and W; "
                         "no GPU needed)")
    ap.add_argument("--bench-log", default=None, metavar="LOG",
                    help="with --trace-summary-from: the profiled bench.py's output, for its HIP-event figures")
    ap.add_argument("--counters-from", default=None, metavar="DIR",
                    help="write profiles/<workload>_counters.{json,md} from the rocprofv3 runs under DIR "
                         "(trace/, pmc1..pmc4; see WORKLOAD_CMDS) with --calibration-from CAL (no GPU needed); "
                         "for the step workload also profiles/traffic.json")
    ap.add_argument("--calibration-from", default=None, metavar="CAL")
    args = ap.parse_args()
    if args.counters_from:
        from exact_io_aware_51_amd import workloads as W
        write_counter_report(args.counters_from, W.WORKLOADS[args.workload], args.calibration_from)
        return
    if args.trace_summary_from:
        from exact_io_aware_51_amd import workloads as W
        write_trace_summary(args.trace_summary_from, W.WORKLOADS[args.workload], args.warmup, args.steps,
                            args.bench_log)
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "the attention path shards (batch, head) pairs across GPUs with no communication, "
              "so there is no multi-GPU step to time here.", file=sys.stderr)
        sys.exit(2)

    import torch

    from exact_io_aware_51_amd import workloads as W
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    if args.copy_calibration:
        n = args.copy_calibration * (1 << 20) // 4
        x = torch.ones(n, dtype=torch.float32, device=dev)
        y = torch.empty_like(x)
        for _ in range(5):
            y.copy_(x)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": n * 4, "copy_bytes_written": n * 4, "launches": 5}), flush=True)
        return
    if args.variants:
        print(json.dumps(time_variants(dev)), flush=True)
        return
    if args.sweep:
        print(json.dumps(time_sweep(dev)), flush=True)
        return
    if args.fwd_workload:
        res = time_fwd_only(args.fwd_workload, dev, iters=args.steps, warmup=args.warmup)
        res["workload"] = args.fwd_workload
        print(json.dumps(res), flush=True)
        return
    w = W.WORKLOADS[args.workload]
    if w.mode != "fwd+bwd":
        raise SystemExit(f"workload {w.name} has no backward; the step needs fwd+bwd")
    log(f"bench: workload {w.name} {w.dtype} B={w.B} H={w.H} N={w.N} d={w.d} causal={w.causal}")
    r = Runner(w, dev)
    # fa_bwd's own sequence: dQ (forming the row sums D on the way), then dK/dV
    stages = [("fwd", r.fwd), ("bwd_dq", r.dq_rowsum), ("bwd_dkdv", r.dkdv)]

    for _ in range(args.warmup):
        for _, f in stages:
            f()
    torch.cuda.synchronize()
    K = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)] for _ in range(K)]
    t0 = time.perf_counter()
    for s in range(K):
        ev[s][0].record()
        for i, (_, f) in enumerate(stages):
            f()
            ev[s][i + 1].record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    wall = t1 - t0
    models = kernel_models(w)
    step_flops = sum(m["flops"] for m in models.values())
    kernels = {}
    for i, (name, _) in enumerate(stages):
        times = [ev[s][i].elapsed_time(ev[s][i + 1]) for s in range(K)]
        ms = sum(times) / K
        m = models[name]
        kernels[name] = {"ms": round(ms, 4), **_spread(times), "tflops": round(m["flops"] / (ms * 1e-3) / 1e12, 1),
                         "gbs": round(m["bytes"] / (ms * 1e-3) / 1e9, 1)}
    event_ms = sum(ev[s][0].elapsed_time(ev[s][-1]) for s in range(K)) / K
    dom = max(kernels, key=lambda n: kernels[n]["ms"])
    dm = models[dom]
    dom_ms = kernels[dom]["ms"]
    mfma_bound = dm["flops"] / dm["bytes"] > PEAK_TFLOPS[w.dtype] * 1e12 / (PEAK_HBM_GBS * 1e9)
    if mfma_bound:
        ach = dm["flops"] / (dom_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(ach, 1), "peak": PEAK_TFLOPS[w.dtype], "unit": "TFLOP/s",
                "frac": round(ach / PEAK_TFLOPS[w.dtype], 4)}
    else:
        ach = dm["bytes"] / (dom_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(ach / PEAK_HBM_GBS, 4)}
    roof["traffic"] = traffic_for(dom)
    roof["kernel"] = dom
    roof["algorithmic_per_launch"] = {"flops": dm["flops"], "bytes": dm["bytes"]}

    out = {
        "metric": METRIC,
        "value": round(step_flops * K / wall / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(wall / K * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": f"{w.name}: fwd+bwd, {w.dtype}, B={w.B} H={w.H} N={w.N} d={w.d}, "
                               f"{'causal' if w.causal else 'non-causal'}, seeded N(0,1) Q/K/V/dO",
                   "B": w.B, "H": w.H, "N": w.N, "d": w.d, "causal": w.causal,
                   "parallelism": "single GPU; (batch, head) pairs would shard across GPUs"},
        "frac_of_peak": round(step_flops * K / wall / 1e12 / PEAK_TFLOPS[w.dtype], 4),
        "event_ms_per_step": round(event_ms, 4),
        "kernels": kernels,
        "roofline": roof,
    }
    if not args.no_fwd_workloads:
        fw = {}
        for name in ("c1", "c2", "c3", "c4"):
            log(f"bench: forward-only {name}")
            fw[name] = time_fwd_only(name, dev)
        fw["c5"] = {"ms": kernels["fwd"]["ms"], "tflops": kernels["fwd"]["tflops"],
                    "frac_of_peak": round(kernels["fwd"]["tflops"] / PEAK_TFLOPS[w.dtype], 4)}
        out["fwd_workloads"] = fw
        f8 = {}
        for name in ("c3", "c4"):
            for fmt in ("e4m3", "e5m2"):
                log(f"bench: forward-only {name} shape on {fmt.upper()} inputs")
                f8[name if fmt == "e4m3" else f"{name}_e5m2"] = time_fwd_fp8(name, dev, fmt=fmt)
        out["fwd_fp8_workloads"] = f8
        log("bench: shader clock under the c4 forward")
        clk = clock_under_load("c4", dev)
        if clk is not None:
            clk["c4_frac_of_peak_at_this_clock"] = round(
                fw["c4"]["tflops"] / (PEAK_TFLOPS["bf16"] * clk["gfx_mhz_mean"] / 2400.0), 4)
        out["clock"] = clk
        log("bench: vendor GEMM rate on this GPU (context)")
        out["matmul_ceiling"] = matmul_ceiling(dev)
    if not args.no_cpu_baseline:
        log("bench: timing the CPU oracle")
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
