"""Collects the rocprofv3 evidence behind bench.py's roofline figures.

Runs, each as its own child process under rocprofv3 (this script itself never
touches the GPU):
  1. --kernel-trace --stats over `bench.py --profile-only` (the timed step loop):
     per-kernel average durations;
  2. --pmc FETCH_SIZE, then --pmc WRITE_SIZE, over the same command, and over
     `bench.py --copy-only 1024` (a plain 1 GiB device copy) to calibrate the two
     counters against a known byte count;
  3. --pmc passes of SQ/GRBM counters over the same command (matrix-pipe busy
     cycles, VALU activity, LDS waits and bank conflicts, shader clock);
  4. steps 1 and 3 again for the FP8 kernel without the LSE (Lean P
     probabilities, row sums on the matrix pipe), the BF16 kernel with the LSE,
     the FP8 kernel with the LSE on the MLA shape at 32K, and the exact-channel
     FP8 kernel with the LSE on the Mistral-shaped 16K workload, each looped alone
     by `bench.py --profile-only --profile-kernel`.
The shader clock is derived from GRBM_GUI_ACTIVE (summed over the 8 XCDs) divided
by the kernel's duration from the kernel-trace pass: the dispatch timestamps of
the counter-collection passes include the profiler's start and stop around each
dispatch and run about 10% longer, which is why a clock taken over them reads low;
both figures are written.
It writes short text summaries plus traffic.json into OUTDIR (which is then
copied into profiles/).  Raw rocprofv3 output stays in RAWDIR.

Usage: python profile_bench.py [OUTDIR] [RAWDIR]
"""
from __future__ import annotations

import csv
import json
import re
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)
from bench import kernel_source_sha  # noqa: E402

TAG = "attn_fwd_fp8_d128_lse_gauss32k"
# the FP8 d128 kernel with LSE (template: FP8, d_qk, key tile, waves, LSE mode, exact
# channels, float32 Q)
KERNEL = "attn_fwd_kernel<true, 128, 128, 8, 1, false, false>"
KERNEL_RE = re.compile(r"attn_fwd_kernel<true, 128, 128, 8, 1, false, false>")
# kernel trace: the same step loop bench.py times; counter passes: a shorter loop
BENCH_KT = ["python", "bench.py", "--profile-only", "--steps", "20", "--warmup", "5"]
BENCH = ["python", "bench.py", "--profile-only", "--steps", "3", "--warmup", "1"]
COPY_MIB = 1024
COPY = ["python", "bench.py", "--copy-only", str(COPY_MIB)]
# the other two kernels of the metric: (tag, name pattern, profile-kernel choice, title)
OTHERS = [
    ("attn_fwd_fp8_d128_gauss32k", re.compile(r"attn_fwd_kernel<true, 128, 128, 8, 0, false, false>"),
     "fp8", "FP8 attention without the LSE (Lean P), gauss32k (B=1 Hq=32 Hkv=8 N=32768 d=128)",
     4.0 * 32 * 32768.0 ** 2 * 128 / 2),
    ("attn_fwd_bf16_d128_lse_gauss32k", re.compile(r"attn_fwd_kernel<false, 128, 64, 8, 1, false, false>"),
     "bf16", "BF16 attention with the LSE, gauss32k (B=1 Hq=32 Hkv=8 N=32768 d=128)",
     4.0 * 32 * 32768.0 ** 2 * 128 / 2),
    ("attn_fwd_fp8_d192_lse_mla32k", re.compile(r"attn_fwd_kernel<true, 192, 128, 8, 1, false, false>"),
     "fp8_mla32k", "FP8 attention with the LSE, mla32k (B=1 H=16 N=32768 d_qk=192 d_v=128)",
     2.0 * 16 * 32768.0 ** 2 * 320 / 2),
    ("attn_fwd_fp8_outliers_d128_lse_mistral16k",
     re.compile(r"attn_fwd_kernel<true, 128, 128, 8, 1, true, false>"), "fp8_outliers_mistral16k",
     "exact-channel FP8 attention with the LSE, mistral16k (B=1 Hq=32 Hkv=8 N=16384 d=128)",
     4.0 * 32 * 16384.0 ** 2 * 128 / 2),
]
SQ_PASSES = [
    ["SQ_WAVE_CYCLES", "SQ_BUSY_CYCLES", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_ACTIVE_INST_VALU",
     "SQ_VALU_MFMA_COEXEC_CYCLES", "SQ_WAIT_INST_LDS", "SQ_WAIT_ANY", "GRBM_GUI_ACTIVE"],
    ["SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_LDS", "SQ_LDS_BANK_CONFLICT",
     "SQ_ACTIVE_INST_LDS", "SQ_INSTS_SALU", "SQ_INSTS_VALU_TRANS_F32", "SQ_ACTIVE_INST_ANY"],
]


def run(cmd, log, timeout=240):
    print("+", " ".join(cmd), flush=True)
    with open(log, "w") as f:
        r = subprocess.run(cmd, stdout=f, stderr=subprocess.STDOUT, cwd=ROOT, timeout=timeout)
    if r.returncode != 0:
        raise SystemExit(f"command failed ({r.returncode}): {' '.join(cmd)}; see {log}")


def rocprof(args, prog, raw, name):
    d = os.path.join(raw, name)
    cmd = ["rocprofv3", *args, "-d", d, "-o", "run", "--output-format", "csv", "--", *prog]
    run(cmd, os.path.join(raw, name + ".log"))
    return d, " ".join(cmd)


def counters(d, match):
    """{dispatch: {counter: value}} and {dispatch: duration_ns} for kernels whose
    name matches `match` (a compiled pattern or a lower-case substring)."""
    vals, dur = {}, {}
    with open(os.path.join(d, "run_counter_collection.csv")) as f:
        for r in csv.DictReader(f):
            name = r["Kernel_Name"]
            if not (match.search(name) if hasattr(match, "search") else match in name.lower()):
                continue
            i = int(r["Dispatch_Id"])
            vals.setdefault(i, {}).setdefault(r["Counter_Name"], 0.0)
            vals[i][r["Counter_Name"]] += float(r["Counter_Value"])
            dur[i] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    return vals, dur


def mean_over(vals, key):
    xs = [v[key] for v in vals.values() if key in v]
    return sum(xs) / len(xs)


def sq_summary(prog, kre, raw, name, title, path, trace_ns=None):
    """SQ/GRBM counter passes over `prog` for the kernels matching `kre`, summarised
    (means per dispatch plus derived ratios) into `path`; trace_ns: the kernel's average
    duration from its kernel-trace pass (the clock's denominator)."""
    agg, cmdl = {}, []
    for i, p in enumerate(SQ_PASSES):
        d, c = rocprof(["--pmc", *p], prog, raw, f"{name}{i}")
        cmdl.append(c)
        v, dur = counters(d, kre)
        for k in p:
            agg[k] = mean_over(v, k)
        agg.setdefault("dur_ns", sum(dur.values()) / len(dur))
    xcd, cus, simds = 8, 256, 4
    gui = agg["GRBM_GUI_ACTIVE"] / xcd                     # cycles per XCD
    sclk_pmc = gui / agg["dur_ns"] * 1e3
    sclk = gui / trace_ns * 1e3 if trace_ns else sclk_pmc
    simd_cycles = gui * cus * simds
    lines = [f"# SQ/GRBM counters, {title} (means per dispatch)"]
    lines += [f"# command: {c}" for c in cmdl]
    lines += [f"{k:32s} {v:16.0f}" for k, v in agg.items()]
    lines += ["", "derived:",
              f"  shader clock             {sclk:8.0f} MHz (GRBM_GUI_ACTIVE / {xcd} XCDs / "
              f"kernel-trace duration {trace_ns / 1e3 if trace_ns else float('nan'):.1f} us)",
              f"  (over the counter pass's own dispatch duration {agg['dur_ns'] / 1e3:.1f} us, "
              f"which includes the profiler's start/stop: {sclk_pmc:.0f} MHz)",
              f"  MFMA pipe busy           {agg['SQ_VALU_MFMA_BUSY_CYCLES'] / simd_cycles:8.3f} "
              f"of SIMD cycles",
              f"  VALU co-issued with MFMA {agg['SQ_VALU_MFMA_COEXEC_CYCLES'] / agg['SQ_VALU_MFMA_BUSY_CYCLES']:8.3f} "
              f"of MFMA-busy cycles",
              f"  VALU instr per MFMA      {agg['SQ_INSTS_VALU'] / agg['SQ_INSTS_MFMA']:8.2f}",
              f"  LDS instr per MFMA       {agg['SQ_INSTS_LDS'] / agg['SQ_INSTS_MFMA']:8.2f}",
              f"  LDS bank-conflict cycles per LDS instr "
              f"{agg['SQ_LDS_BANK_CONFLICT'] / agg['SQ_INSTS_LDS']:8.2f}",
              f"  LDS wait / wave cycles   {agg['SQ_WAIT_INST_LDS'] / agg['SQ_WAVE_CYCLES']:8.3f}"]
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")


def main() -> int:
    out = sys.argv[1] if len(sys.argv) > 1 else os.path.join(ROOT, "gpurun_out", "profiles")
    raw = sys.argv[2] if len(sys.argv) > 2 else os.path.join(ROOT, "gpurun_out", "rocprof_raw")
    os.makedirs(out, exist_ok=True)
    os.makedirs(raw, exist_ok=True)

    # 1. kernel trace + stats
    d, cmd = rocprof(["--kernel-trace", "--stats"], BENCH_KT, raw, "kt")
    with open(os.path.join(d, "run_kernel_stats.csv")) as f:
        rows = list(csv.DictReader(f))
    lines = [f"# rocprofv3 kernel statistics: FP8 causal attention step, gauss32k "
             f"(B=1 Hq=32 Hkv=8 N=32768 d=128)", f"# command: {cmd}",
             f"# kernel source sha: {kernel_source_sha()}", "",
             f"{'kernel':70s} {'calls':>6s} {'avg_us':>10s} {'min_us':>10s} {'max_us':>10s} {'pct':>6s}"]
    attn_avg_ns = None
    kernel_name = KERNEL
    for r in rows:
        name = r["Name"]
        lines.append(f"{name[:70]:70s} {int(r['Calls']):6d} {float(r['AverageNs'])/1e3:10.1f} "
                     f"{float(r['MinNs'])/1e3:10.1f} {float(r['MaxNs'])/1e3:10.1f} "
                     f"{float(r['Percentage']):6.2f}")
        if KERNEL_RE.search(name):
            attn_avg_ns = float(r["AverageNs"])
            kernel_name = name
    flops = 4.0 * 32 * 32768.0 ** 2 * 128 / 2
    if attn_avg_ns:
        lines += ["", f"attention kernel average {attn_avg_ns/1e3:.1f} us -> "
                      f"{flops / attn_avg_ns / 1e3:.1f} TFLOP/s (causal FLOPs {flops:.4e})"]
    with open(os.path.join(out, f"{TAG}_kernel_stats.txt"), "w") as f:
        f.write("\n".join(lines) + "\n")

    # 2. HBM bytes: FETCH_SIZE and WRITE_SIZE (KiB per dispatch), calibrated on a copy
    res = {}
    cmds = {}
    for ctr in ("FETCH_SIZE", "WRITE_SIZE"):
        d, cmds[f"attn_{ctr}"] = rocprof(["--pmc", ctr], BENCH, raw, f"attn_{ctr}")
        v, _ = counters(d, KERNEL_RE)
        res[f"attn_{ctr}_kib"] = mean_over(v, ctr)
        d, cmds[f"copy_{ctr}"] = rocprof(["--pmc", ctr], COPY, raw, f"copy_{ctr}")
        v, _ = counters(d, "copy")
        res[f"copy_{ctr}_kib"] = max(x[ctr] for x in v.values())
    copy_bytes = COPY_MIB * 2.0 ** 20
    f_fetch = copy_bytes / (res["copy_FETCH_SIZE_kib"] * 1024)
    f_write = copy_bytes / (res["copy_WRITE_SIZE_kib"] * 1024)
    fetch_b = res["attn_FETCH_SIZE_kib"] * 1024 * f_fetch
    write_b = res["attn_WRITE_SIZE_kib"] * 1024 * f_write
    alg = 32768 * 32 * 128 + 2 * 32768 * 8 * 128 + 32768 * 32 * 128 * 2 + 32 * 32768 * 4
    traffic = {TAG: {"source_sha": kernel_source_sha(), "kernel": kernel_name,
                     "hbm_bytes_per_launch": round(fetch_b + write_b),
                     "fetch_bytes": round(fetch_b), "write_bytes": round(write_b),
                     "algorithmic_bytes": alg,
                     "calibration": {"copy_mib": COPY_MIB, "fetch_factor": round(f_fetch, 4),
                                     "write_factor": round(f_write, 4)},
                     "raw_kib": res, "commands": cmds}}
    with open(os.path.join(out, "traffic.json"), "w") as f:
        json.dump(traffic, f, indent=1)
    with open(os.path.join(out, f"{TAG}_traffic.txt"), "w") as f:
        f.write(f"# HBM traffic per launch of {kernel_name} (gauss32k, with LSE)\n")
        for k, c in cmds.items():
            f.write(f"# {k}: {c}\n")
        f.write(f"copy of {COPY_MIB} MiB: FETCH_SIZE {res['copy_FETCH_SIZE_kib']:.0f} KiB, "
                f"WRITE_SIZE {res['copy_WRITE_SIZE_kib']:.0f} KiB -> factors "
                f"{f_fetch:.4f} / {f_write:.4f}\n")
        f.write(f"attention: FETCH_SIZE {res['attn_FETCH_SIZE_kib']:.0f} KiB, WRITE_SIZE "
                f"{res['attn_WRITE_SIZE_kib']:.0f} KiB per launch\n")
        f.write(f"calibrated: read {fetch_b/2**20:.1f} MiB + write {write_b/2**20:.1f} MiB = "
                f"{(fetch_b + write_b)/2**20:.1f} MiB; algorithmic (Q, K, V read once, O and "
                f"LSE written once) {alg/2**20:.1f} MiB\n")

    # 3. SQ / GRBM counters
    sq_summary(BENCH, KERNEL_RE, raw, "sq", f"{kernel_name}, gauss32k with LSE",
               os.path.join(out, f"{TAG}_counters.txt"), trace_ns=attn_avg_ns)

    # 4. the FP8 kernel without the LSE and the BF16 kernel with it
    for tag, kre, choice, title, kflops in OTHERS:
        prog_kt = BENCH_KT + ["--profile-kernel", choice]
        prog = BENCH + ["--profile-kernel", choice]
        d, cmd = rocprof(["--kernel-trace", "--stats"], prog_kt, raw, f"kt_{choice}")
        with open(os.path.join(d, "run_kernel_stats.csv")) as f:
            rows = list(csv.DictReader(f))
        name, avg = None, None
        for r in rows:
            if kre.search(r["Name"]):
                name, avg = r["Name"], float(r["AverageNs"])
        lines = [f"# rocprofv3 kernel statistics: {title}, the kernel looped alone",
                 f"# command: {cmd}", f"# kernel source sha: {kernel_source_sha()}", "",
                 f"{'kernel':70s} {'calls':>6s} {'avg_us':>10s} {'min_us':>10s} {'max_us':>10s} "
                 f"{'pct':>6s}"]
        for r in rows:
            lines.append(f"{r['Name'][:70]:70s} {int(r['Calls']):6d} "
                         f"{float(r['AverageNs'])/1e3:10.1f} {float(r['MinNs'])/1e3:10.1f} "
                         f"{float(r['MaxNs'])/1e3:10.1f} {float(r['Percentage']):6.2f}")
        if avg:
            lines += ["", f"kernel average {avg/1e3:.1f} us -> {kflops / avg / 1e3:.1f} TFLOP/s"]
        with open(os.path.join(out, f"{tag}_kernel_stats.txt"), "w") as f:
            f.write("\n".join(lines) + "\n")
        sq_summary(prog, kre, raw, f"sq_{choice}", f"{name} ({title})",
                   os.path.join(out, f"{tag}_counters.txt"), trace_ns=avg)
    print("profile summaries written to", out, flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
