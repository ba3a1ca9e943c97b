"""Benchmark of the causal prefill attention hot path on one MI355X.

One step = the whole FP8 path over one batch of the "gauss32k" workload
(B=1, Hq=32, Hkv=8, N=32768, d=128, iid N(0,1) inputs already resident in
HBM as float32): quantize_e4m3 of Q, K and V (per-tensor scales), then
attn_fwd_causal_fp8 writing O (bf16) and the LSE.  `value` is causal TFLOP/s
of that step, counting only the attention FLOPs 4*B*Hq*N^2*d/2.

Also printed (in "extra"): the attention kernels alone, FP8 with and without
the LSE, BF16, and the MLA shape at 32K, each timed with HIP events on the
stream the kernels run on.  `roofline` is for the dominant kernel (the FP8
attention kernel): achieved = algorithmic FLOPs per launch / its mean launch
time; `cpu_baseline` times the fp64 CPU oracle on a bounded sample.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--no-extra]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import subprocess
import sys
import threading
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "causal prefill attn TFLOP/s @32K (FP8/BF16, d128 & MLA); % MFMA peak"
PEAK_TFLOPS = {"fp8": 5000.0, "bf16": 2500.0}   # MI355X dense MFMA peaks
PAGES_FP8_D128_32K = 2672.0                      # the pages' figure (context)


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


class ClockPoller:
    """Samples the GPU shader clock with amd-smi while the timed loop runs."""

    def __init__(self, period: float = 0.05):
        self.period = period
        self.samples: list[float] = []
        self._stop = threading.Event()
        self._t = None

    def _read(self) -> float | None:
        try:
            r = subprocess.run(["amd-smi", "metric", "-g", "0", "-c", "--json"],
                               capture_output=True, text=True, timeout=5)
            data = json.loads(r.stdout)
            if isinstance(data, list):
                data = data[0]
            clk = data.get("clock", data)
            gfx = clk.get("gfx_0") or clk.get("GFX_0") or {}
            val = gfx.get("clk")
            if isinstance(val, dict):
                val = val.get("value")
            return float(val) if val not in (None, "N/A") else None
        except Exception:
            return None

    def _run(self):
        while not self._stop.is_set():
            v = self._read()
            if v is not None:
                self.samples.append(v)
            self._stop.wait(self.period)

    def __enter__(self):
        self._t = threading.Thread(target=self._run, daemon=True)
        self._t.start()
        return self

    def __exit__(self, *a):
        self._stop.set()
        self._t.join(timeout=10)

    def mean(self):
        return sum(self.samples) / len(self.samples) if self.samples else None


def time_events(fn, iters: int, warmup: int = 2):
    """Mean duration (ms) of fn() over `iters` launches, from HIP events on the
    current stream (the stream the library launches on)."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(iters)]
    for a, b in evs:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    return sum(a.elapsed_time(b) for a, b in evs) / iters


def kernel_source_sha() -> str:
    h = hashlib.sha256()
    for name in ("attn_fwd.hip", "kernels.h"):
        with open(os.path.join(ROOT, "bf16_causal_prefill_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_from_profile(kernel_tag: str):
    """HBM bytes per launch from the committed counter summary, if it was taken
    on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            data = json.load(f)
        ent = data[kernel_tag]
        if ent.get("source_sha") != kernel_source_sha():
            return None
        return ent["hbm_bytes_per_launch"]
    except Exception:
        return None


def cpu_baseline(w, x, n_heads: int):
    """fp64 oracle on the first `n_heads` query heads (all N rows) of the
    workload's e4m3-decoded inputs; returns the baseline object."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    G = w.Hq // w.Hkv
    n_kv = (n_heads + G - 1) // G
    dec = {}
    for n in "qkv":
        codes, ds = oracle.quantize_e4m3(x[n], per_head=w.fp8_per_head)
        dsb = ds[None, None, :, None] if w.fp8_per_head else ds[0]
        sl = slice(0, n_heads) if n == "q" else slice(0, n_kv)
        dec[n] = oracle.e4m3_decode(codes[:, :, sl]) * (dsb[:, :, sl] if w.fp8_per_head else dsb)
    t0 = time.perf_counter()
    oracle.causal_attention(dec["q"], dec["k"], dec["v"], w.softmax_scale)
    dt = time.perf_counter() - t0
    flops = 2.0 * w.B * n_heads * float(w.N) ** 2 * (w.d_qk + w.d_v) / 2.0
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle", "seconds": round(dt, 2),
            "sample": f"{w.name}: query heads 0..{n_heads - 1} of {w.Hq} (KV heads 0..{n_kv - 1}), "
                      f"all {w.N} rows, e4m3-decoded inputs in float64; "
                      f"throughput scaled by the sample's causal FLOPs"}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="gauss32k")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-extra", action="store_true")
    ap.add_argument("--cpu-heads", type=int, default=8)
    ap.add_argument("--profile-only", action="store_true",
                    help="run the step loop only (for rocprofv3), no JSON line")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on one GPU only: the kernels take one GPU's share of the "
              "work and no figure at several GPUs is produced (use --gpus 1)", file=sys.stderr)
        return 2

    import numpy as np
    import torch
    import bf16_causal_prefill_amd as ba
    import workloads

    ba.load_library()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = "cuda:0"
    w = workloads.get(args.workload)
    log(f"bench: generating {w.name} inputs")
    x = workloads.generate(w)
    xd = {n: torch.from_numpy(x[n]).to(dev) for n in "qkv"}
    nds = lambda H: (H if w.fp8_per_head else 1)
    codes = {n: torch.empty(x[n].shape, device=dev, dtype=torch.uint8) for n in "qkv"}
    ds = {"q": torch.empty(nds(w.Hq), device=dev), "k": torch.empty(nds(w.Hkv), device=dev),
          "v": torch.empty(nds(w.Hkv), device=dev)}
    o = torch.empty((w.B, w.N, w.Hq, w.d_v), device=dev, dtype=torch.bfloat16)
    lse = torch.empty((w.B, w.Hq, w.N), device=dev, dtype=torch.float32)
    flops = workloads.causal_flops(w)

    def quant():
        for n in "qkv":
            ba.quantize_e4m3(xd[n], codes[n], ds[n], per_head=w.fp8_per_head)

    def attn_fp8(with_lse=True):
        ba.attn_fwd_causal_fp8(codes["q"], codes["k"], codes["v"], ds["q"], ds["k"], ds["v"],
                               o, lse if with_lse else None, softmax_scale=w.softmax_scale,
                               descale_per_head=int(w.fp8_per_head))

    ev_attn = []

    def step():
        quant()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        attn_fp8(True)
        b.record()
        ev_attn.append((a, b))

    log(f"bench: warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev_attn.clear()
    log(f"bench: timing {args.steps} steps")
    with ClockPoller() as clk:
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            step()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
    if args.profile_only:
        log("bench: profile-only run done")
        return 0
    ms_step = (t1 - t0) * 1e3 / args.steps
    attn_ms = sum(a.elapsed_time(b) for a, b in ev_attn) / len(ev_attn)
    value = flops / (ms_step * 1e-3) / 1e12
    achieved = flops / (attn_ms * 1e-3) / 1e12
    log(f"bench: step {ms_step:.3f} ms ({value:.1f} TFLOP/s); fp8 attention {attn_ms:.3f} ms "
        f"({achieved:.1f} TFLOP/s)")

    extra = {}
    if not args.no_extra:
        extra["fp8_attn_lse_ms"] = round(attn_ms, 4)
        t = time_events(lambda: attn_fp8(False), 10)
        extra["fp8_attn_nolse_ms"] = round(t, 4)
        extra["fp8_attn_nolse_tflops"] = round(flops / t / 1e9, 1)
        t = time_events(quant, 10)
        extra["quantize_qkv_ms"] = round(t, 4)
        qbytes = sum(x[n].nbytes * 2 + x[n].size for n in "qkv")  # 2 reads + code write
        extra["quantize_qkv_GBps"] = round(qbytes / t / 1e6, 1)
        # BF16 on the same workload
        xb = {n: xd[n].to(torch.bfloat16) for n in "qkv"}
        t = time_events(lambda: ba.attn_fwd_causal_bf16(xb["q"], xb["k"], xb["v"], o, lse,
                                                        softmax_scale=w.softmax_scale), 10)
        extra["bf16_attn_ms"] = round(t, 4)
        extra["bf16_attn_tflops"] = round(flops / t / 1e9, 1)
        extra["bf16_pct_peak"] = round(100 * flops / t / 1e9 / PEAK_TFLOPS["bf16"], 2)
        del xb
        # MLA shape at 32K
        wm = workloads.get("mla32k")
        log("bench: generating mla32k inputs")
        xm = workloads.generate(wm)
        xmd = {n: torch.from_numpy(xm[n]).to(dev) for n in "qkv"}
        om = torch.empty((wm.B, wm.N, wm.Hq, wm.d_v), device=dev, dtype=torch.bfloat16)
        lm = torch.empty((wm.B, wm.Hq, wm.N), device=dev, dtype=torch.float32)
        fm = workloads.causal_flops(wm)
        cm = {n: torch.empty(xm[n].shape, device=dev, dtype=torch.uint8) for n in "qkv"}
        dm = {n: torch.empty(xm[n].shape[2], device=dev) for n in "qkv"}
        for n in "qkv":
            ba.quantize_e4m3(xmd[n], cm[n], dm[n], per_head=True)
        t = time_events(lambda: ba.attn_fwd_causal_fp8(cm["q"], cm["k"], cm["v"], dm["q"],
                                                       dm["k"], dm["v"], om, lm,
                                                       softmax_scale=wm.softmax_scale,
                                                       descale_per_head=1), 10)
        extra["mla32k_fp8_attn_tflops"] = round(fm / t / 1e9, 1)
        t = time_events(lambda: ba.attn_fwd_causal_fp8(cm["q"], cm["k"], cm["v"], dm["q"],
                                                       dm["k"], dm["v"], om, None,
                                                       softmax_scale=wm.softmax_scale,
                                                       descale_per_head=1), 10)
        extra["mla32k_fp8_attn_nolse_tflops"] = round(fm / t / 1e9, 1)
        xmb = {n: xmd[n].to(torch.bfloat16) for n in "qkv"}
        t = time_events(lambda: ba.attn_fwd_causal_bf16(xmb["q"], xmb["k"], xmb["v"], om, lm,
                                                        softmax_scale=wm.softmax_scale), 10)
        extra["mla32k_bf16_attn_tflops"] = round(fm / t / 1e9, 1)
        del xmd, xmb, cm

    cpu = None
    if not args.no_cpu:
        log(f"bench: timing the CPU oracle on {args.cpu_heads} heads")
        cpu = cpu_baseline(w, x, args.cpu_heads)

    sclk = clk.mean()
    rec = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": round(value / PAGES_FP8_D128_32K, 4),
        "dtype": "fp8_e4m3",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "N": w.N,
                   "d_qk": w.d_qk, "d_v": w.d_v,
                   "step": "quantize_e4m3(q,k,v) + attn_fwd_causal_fp8 (O + LSE)",
                   "parallelism": "single GPU"},
        "pct_peak": round(100 * value / PEAK_TFLOPS["fp8"], 2),
        "sclk_mhz": round(sclk, 1) if sclk else None,
        "roofline": {"bound": "mfma", "kernel": "attn_fwd_kernel<fp8,d128>",
                     "achieved": round(achieved, 2), "peak": PEAK_TFLOPS["fp8"],
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_TFLOPS["fp8"], 4),
                     "traffic": traffic_from_profile("attn_fwd_fp8_d128_gauss32k")},
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
