"""Benchmark of the causal prefill attention hot path on one MI355X.

One step = the whole FP8 path over one batch of the "gauss32k" workload
(B=1, Hq=32, Hkv=8, N=32768, d=128, iid N(0,1) inputs already resident in HBM
as float32): quantize_e4m3_qkv, which quantises K and V with their absmax scales and Q
with the per-tensor scale that makes the FP8 softmax constant a power of two (the codes
of quantize_e4m3 and quantize_e4m3_q_pow2, in four kernels instead of twelve), then
attn_fwd_causal_fp8 writing O (bf16) and the LSE (fp32).  `value` is the causal
TFLOP/s of that step, counting only the attention FLOPs 4*B*Hq*N^2*d/2.

`roofline` describes the dominant kernel (the FP8 attention kernel): achieved =
its algorithmic FLOPs per launch / its mean launch time, measured with HIP
events on the stream the library launches on, over the timed steps; peak = the
MI355X dense FP8 matrix peak; traffic = HBM bytes per launch from the committed
rocprofv3 counter summary when it was taken on the current kernel source, else
null.  `sclk_mhz` is the shader clock sampled from the device while the FP8
kernel runs back to back, and `frac_of_clock_adjusted_peak` the kernel's rate
against the peak at that clock.  `cpu_baseline` times the fp64 CPU oracle on a
bounded sample of the same workload.  "extra" holds the other precisions and
shapes of the metric (FP8 with and without the LSE, BF16, the MLA shape at 32K)
timed the same way, the step from float32 Q (the attention kernel encoding Q as it
loads it, after a quantiser pass that writes Q's descales only) beside the step
above, the energy per FLOP of the attention kernels from the
device's energy counter, and the entry points past the pages' scope (Hadamard
pre-step, chunked prefill with a query offset, the merge of partial attentions,
the flash_attn_func wrapper).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--no-extra]
       python bench.py --profile-only [--steps K]   (step loop only, for rocprofv3)
       python bench.py --profile-only --profile-kernel fp8|bf16
                                                    (loop of the FP8 attention without the LSE,
                                                     or of the BF16 attention with it)
       python bench.py --copy-only MIB              (plain device copy, counter calibration)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import threading
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "causal prefill attn TFLOP/s @32K (FP8/BF16, d128 & MLA); % MFMA peak"
# MI355X dense matrix peaks (TFLOP/s): 256 CUs x 2.4 GHz x 8192 (fp8) / 4096 (bf16).
PEAK_TFLOPS = {"fp8": 5000.0, "bf16": 2500.0}
PAGES_FP8_D128_32K = 2672.0   # the pages' MI355X figure (B, H unstated): context only
KERNEL_SOURCES = ("attn_fwd.h", "attn_fwd_fp8.hip", "attn_common.h", "kernels.h")


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def kernel_source_sha() -> str:
    """Hash of the attention kernel sources; the committed counter summary is
    used only when it was taken on exactly these sources."""
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "bf16_causal_prefill_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_from_profile(tag: str):
    """HBM bytes per launch of kernel `tag` from profiles/traffic.json, or None."""
    try:
        with open(os.path.join(ROOT, "profiles", "traffic.json")) as f:
            ent = json.load(f)[tag]
        if ent.get("source_sha") != kernel_source_sha():
            return None
        return ent["hbm_bytes_per_launch"]
    except Exception:
        return None


def time_events(fn, iters: int, warmup: int = 2) -> float:
    """Median duration (ms) of fn() from HIP events on torch's current stream,
    which is the stream the library launches on (the median, so that one delayed
    launch does not set the figure)."""
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
    ts = sorted(a.elapsed_time(b) for a, b in evs)
    return ts[len(ts) // 2]


def gpu_energy_reader():
    """A function returning (joules, counter timestamp in s) for the GPU's energy
    accumulator (amdsmi: counts times the counter resolution in microjoules; the
    timestamp is when the device last updated it), or None with the reason when it
    is not readable.  Only one visible GPU is supported."""
    try:
        import amdsmi
        amdsmi.amdsmi_init()
        hs = amdsmi.amdsmi_get_processor_handles()
        if len(hs) != 1:
            return None, f"{len(hs)} GPUs visible to amdsmi"
        h = hs[0]

        def read():
            e = amdsmi.amdsmi_get_energy_count(h)
            return (e["energy_accumulator"] * e["counter_resolution"] * 1e-6,
                    e["timestamp"] * 1e-9)
        read()
        return read, None
    except Exception as exc:   # no library, no permission, no counter
        return None, f"{type(exc).__name__}: {exc}"[:120]


def gpu_clock_reader():
    """A function returning the GPU's current shader (gfx) clock in MHz, the mean over
    its XCDs when the device reports one per XCD, or None when not readable."""
    try:
        import amdsmi
        amdsmi.amdsmi_init()
        hs = amdsmi.amdsmi_get_processor_handles()
        if len(hs) != 1:
            return None
        h = hs[0]

        def read():
            m = amdsmi.amdsmi_get_gpu_metrics_info(h)
            vals = m.get("current_gfxclks")
            if isinstance(vals, list):
                vals = [v for v in vals if isinstance(v, (int, float)) and 0 < v < 10000]
                if vals:
                    return sum(vals) / len(vals)
            v = m.get("current_gfxclk")
            return float(v) if isinstance(v, (int, float)) and 0 < v < 10000 else None
        return read if read() is not None else None
    except Exception:
        return None


def energy_of(fn, flops: float, read, seconds: float = 3.0, clock=None) -> dict:
    """Run fn back to back for about `seconds`; the mean power is the energy counter's
    increase over its own timestamps taken inside the loop (after a settling second,
    so both readings fall in steady state), and energy per call = power x the
    measured time per call.  Returns TFLOP/J and the mean power."""
    import torch
    t_ms = time_events(fn, 3)                       # ms per call
    iters = max(20, int(seconds * 1e3 / t_ms))
    settle = max(1, int(1e3 / t_ms))
    torch.cuda.synchronize()
    h0 = time.perf_counter()
    for _ in range(settle):
        fn()
    torch.cuda.synchronize()
    (e0, s0) = read()
    clk, stop = [], threading.Event()

    def poll():                         # the clock every 10 ms until the loop has drained
        while not stop.wait(0.01):
            c = clock()
            if c is not None:
                clk.append(c)
    poller = threading.Thread(target=poll, daemon=True) if clock is not None else None
    if poller is not None:
        poller.start()
    t0 = time.perf_counter()
    for _ in range(iters):
        fn()
    torch.cuda.synchronize()
    if poller is not None:
        stop.set()
        poller.join()
    t1 = time.perf_counter()
    (e1, s1) = read()
    watts = (e1 - e0) / (s1 - s0) if s1 > s0 else None
    per_call_s = (t1 - t0) / iters
    return {"tflop_per_j": round(flops / (watts * per_call_s) / 1e12, 3) if watts else None,
            "avg_w": round(watts, 1) if watts else None, "calls": iters,
            "loop_s": round(t1 - t0, 3), "counter_s": round(s1 - s0, 3),
            "settle_s": round(t0 - h0, 3),
            "sclk_mhz": round(sum(clk) / len(clk), 1) if clk else None}


def timed_with_clock(fn, flops: float, clock=None, seconds: float = 1.0, iters: int = 30):
    """Kernel-only rate of fn: about 0.3 s of back-to-back calls to settle the clock, then
    `iters` calls timed with HIP events on the current stream while a host thread polls
    the shader clock every 5 ms; returns (ms, TFLOP/s, mean SCLK in MHz or None)."""
    import torch
    t_ms = time_events(fn, 3)
    for _ in range(max(2, int(300.0 / max(t_ms, 1e-3)))):
        fn()
    torch.cuda.synchronize()
    n = max(iters, int(seconds * 1e3 / max(t_ms, 1e-3)))
    clk, stop = [], threading.Event()

    def poll():
        while not stop.wait(0.005):
            c = clock()
            if c is not None:
                clk.append(c)
    poller = threading.Thread(target=poll, daemon=True) if clock is not None else None
    if poller is not None:
        poller.start()
    ms = time_events(fn, n, warmup=0)
    if poller is not None:
        stop.set()
        poller.join()
    return ms, flops / ms / 1e9, (round(sum(clk) / len(clk), 1) if clk else None)


def float32_q_lines(ba, w, xd, codes, ds, o, lse, flops) -> dict:
    """The FP8 step with the LSE two ways, timed in alternating rounds: quantize_e4m3_qkv
    writing Q's codes + attn_fwd_causal_fp8, and quantize_e4m3_qkv with Q's descales only
    + attn_fwd_causal_fp8_qf32 (the kernel encodes float32 Q as it loads it; O and LSE
    are byte-identical).  Also the float32-Q attention kernel alone."""
    ph = int(w.fp8_per_head)

    def quant(q_out):
        ba.quantize_e4m3_qkv(xd["q"], xd["k"], xd["v"], q_out, codes["k"], codes["v"],
                             ds["q"], ds["k"], ds["v"], per_head=w.fp8_per_head, q_pow2=True,
                             softmax_scale=w.softmax_scale)

    attn_codes = lambda: ba.attn_fwd_causal_fp8(
        codes["q"], codes["k"], codes["v"], ds["q"], ds["k"], ds["v"], o, lse,
        softmax_scale=w.softmax_scale, descale_per_head=ph)
    attn_f32 = lambda: ba.attn_fwd_causal_fp8_qf32(
        xd["q"], codes["k"], codes["v"], ds["q"], ds["k"], ds["v"], o, lse,
        softmax_scale=w.softmax_scale, descale_per_head=ph)
    runs = {"codes": (lambda: (quant(codes["q"]), attn_codes())),
            "f32": (lambda: (quant(None), attn_f32())), "attn_f32": attn_f32}
    ts = {k: [] for k in runs}
    for _ in range(3):
        for k, fn in runs.items():
            ts[k].append(time_events(fn, 10))
    med = {k: sorted(v)[len(v) // 2] for k, v in ts.items()}
    return {"step_q_codes_ms": round(med["codes"], 4),
            "step_q_float32_ms": round(med["f32"], 4),
            "fp8_lse_q_float32_tflops": round(flops / med["attn_f32"] / 1e9, 1)}


def config_lines(ba, torch, name: str, clock) -> dict:
    """Kernel-only TFLOP/s, % of the dense peak and sustained SCLK of the attention
    kernels on one workload: FP8 with the LSE (Q quantised for the power-of-two softmax
    constant, and with its absmax scale), FP8 without the LSE, BF16 with the LSE; on the
    outlier-channel recipe also the exact-channel kernel on the joint Q/K quantiser's
    codes (the path that meets the LSE gate there) and that quantiser's time."""
    import workloads
    w = workloads.get(name)
    x = workloads.generate(w)
    dev = "cuda:0"
    xd = {n: torch.from_numpy(x[n]).to(dev) for n in "qkv"}
    nds = lambda H: (H if w.fp8_per_head else 1)
    codes = {n: torch.empty(x[n].shape, device=dev, dtype=torch.uint8) for n in "qkv"}
    ds = {"q": torch.empty(nds(w.Hq), device=dev), "k": torch.empty(nds(w.Hkv), device=dev),
          "v": torch.empty(nds(w.Hkv), device=dev)}
    o = torch.empty((w.B, w.N, w.Hq, w.d_v), device=dev, dtype=torch.bfloat16)
    lse = torch.empty((w.B, w.Hq, w.N), device=dev, dtype=torch.float32)
    flops = workloads.causal_flops(w)
    ph = int(w.fp8_per_head)
    out = {}

    def put(tag, fn, prec):
        ms, tf, clk = timed_with_clock(fn, flops, clock)
        out[tag + "_tflops"] = round(tf, 1)
        out[tag + "_pct_peak"] = round(100.0 * tf / PEAK_TFLOPS[prec], 2)
        out[tag + "_sclk_mhz"] = clk

    for n in "kv":
        ba.quantize_e4m3(xd[n], codes[n], ds[n], per_head=w.fp8_per_head)
    ba.quantize_e4m3(xd["q"], codes["q"], ds["q"], per_head=w.fp8_per_head)
    fp8 = lambda L: (lambda: ba.attn_fwd_causal_fp8(
        codes["q"], codes["k"], codes["v"], ds["q"], ds["k"], ds["v"], o, L,
        softmax_scale=w.softmax_scale, descale_per_head=ph))
    put("fp8_lse_absmax_q", fp8(lse), "fp8")
    put("fp8_nolse", fp8(None), "fp8")
    ba.quantize_e4m3_q_pow2(xd["q"], codes["q"], ds["q"], ds["k"], w.softmax_scale,
                            per_head=w.fp8_per_head)
    put("fp8_lse", fp8(lse), "fp8")
    out.update(float32_q_lines(ba, w, xd, codes, ds, o, lse, flops))
    if w.d_qk == 128:
        # the exact-channel kernel (32 channels on the BF16 pipe), on the joint quantiser's
        # codes with the power-of-two Q scale
        perm = torch.empty((w.Hkv, w.d_qk), device=dev, dtype=torch.uint8)
        T = ba.OUTLIER_CHANNELS
        qx = torch.empty((w.B, w.N, w.Hq, T), device=dev, dtype=torch.bfloat16)
        kx = torch.empty((w.B, w.N, w.Hkv, T), device=dev, dtype=torch.bfloat16)
        wsb = torch.empty(ba.quantize_e4m3_qk_outliers_workspace_bytes(w.Hq, w.Hkv, w.d_qk),
                          device=dev, dtype=torch.uint8)
        quant_o = lambda: ba.quantize_e4m3_qk_outliers(
            xd["q"], xd["k"], codes["q"], codes["k"], qx, kx, ds["q"], ds["k"], perm,
            w.fp8_per_head, q_pow2=True, softmax_scale=w.softmax_scale, workspace=wsb)
        t = time_events(quant_o, 10)
        # 2 reads + code write + the side arrays (32 of d channels as bf16)
        qbytes = sum(x[n].nbytes * 2 + x[n].size + x[n].size * 2 * T // w.d_qk for n in "qk")
        out["quantize_qk_outliers_ms"] = round(t, 4)
        out["quantize_qk_outliers_GBps"] = round(qbytes / t / 1e6, 1)
        quant_o()
        fo = lambda L: (lambda: ba.attn_fwd_causal_fp8_outliers(
            codes["q"], codes["k"], codes["v"], qx, kx, ds["q"], ds["k"], ds["v"], o, L,
            softmax_scale=w.softmax_scale, descale_per_head=ph))
        put("fp8_outliers_lse", fo(lse), "fp8")
        put("fp8_outliers_nolse", fo(None), "fp8")
    del codes
    xb = {n: xd[n].to(torch.bfloat16) for n in "qkv"}
    del xd
    put("bf16_lse", lambda: ba.attn_fwd_causal_bf16(xb["q"], xb["k"], xb["v"], o, lse,
                                                    softmax_scale=w.softmax_scale), "bf16")
    return out


def other_workload_loop(ba, torch, choice: str):
    """One call of the attention kernel a profile pass loops on another workload: FP8
    with the LSE on mla32k (Q for the power-of-two constant), or the exact-channel FP8
    kernel with the LSE on mistral16k (the joint quantiser's codes and side arrays)."""
    import workloads
    dev = "cuda:0"
    name = "mla32k" if choice == "fp8_mla32k" else "mistral16k"
    w = workloads.get(name)
    x = workloads.generate(w)
    xd = {n: torch.from_numpy(x[n]).to(dev) for n in "qkv"}
    codes = {n: torch.empty(x[n].shape, device=dev, dtype=torch.uint8) for n in "qkv"}
    ds = {n: torch.empty(x[n].shape[2], device=dev) for n in "qkv"}
    o = torch.empty((w.B, w.N, w.Hq, w.d_v), device=dev, dtype=torch.bfloat16)
    lse = torch.empty((w.B, w.Hq, w.N), device=dev, dtype=torch.float32)
    ba.quantize_e4m3(xd["v"], codes["v"], ds["v"], per_head=True)
    if choice == "fp8_mla32k":
        ba.quantize_e4m3(xd["k"], codes["k"], ds["k"], per_head=True)
        ba.quantize_e4m3_q_pow2(xd["q"], codes["q"], ds["q"], ds["k"], w.softmax_scale,
                                per_head=True)
        return lambda: ba.attn_fwd_causal_fp8(codes["q"], codes["k"], codes["v"], ds["q"],
                                              ds["k"], ds["v"], o, lse,
                                              softmax_scale=w.softmax_scale, descale_per_head=1)
    T = ba.OUTLIER_CHANNELS
    qx = torch.empty((w.B, w.N, w.Hq, T), device=dev, dtype=torch.bfloat16)
    kx = torch.empty((w.B, w.N, w.Hkv, T), device=dev, dtype=torch.bfloat16)
    perm = torch.empty((w.Hkv, w.d_qk), device=dev, dtype=torch.uint8)
    ba.quantize_e4m3_qk_outliers(xd["q"], xd["k"], codes["q"], codes["k"], qx, kx, ds["q"],
                                 ds["k"], perm, True, q_pow2=True, softmax_scale=w.softmax_scale)
    return lambda: ba.attn_fwd_causal_fp8_outliers(codes["q"], codes["k"], codes["v"], qx, kx,
                                                   ds["q"], ds["k"], ds["v"], o, lse,
                                                   softmax_scale=w.softmax_scale,
                                                   descale_per_head=1)


def cpu_baseline(w, x, n_heads: int):
    """The fp64 oracle on query heads 0..n_heads-1 (all N rows) of the workload's
    e4m3-decoded inputs (per-tensor descales from the whole tensors).  Only the
    attention itself is timed; the throughput counts the sample's causal FLOPs."""
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
    dsk = oracle.absmax_descale(x["k"], per_head=False)
    for n, hs in (("k", n_kv), ("v", n_kv), ("q", n_heads)):
        ds = oracle.absmax_descale(x[n], per_head=False)
        if n == "q":      # the Q descale of quantize_e4m3_q_pow2, from the whole tensor
            amax = np.float32(np.max(np.abs(x[n])))
            ds = np.array([oracle.pow2_q_descale_one(amax, dsk[0], w.softmax_scale)],
                          np.float32)
        codes = oracle.encode_with_descale(x[n][:, :, :hs], ds[0])
        dec[n] = oracle.e4m3_decode(codes) * float(ds[0])
    t0 = time.perf_counter()
    oracle.causal_attention(dec["q"], dec["k"], dec["v"], w.softmax_scale)
    dt = time.perf_counter() - t0
    flops = 2.0 * w.B * n_heads * float(w.N) ** 2 * (w.d_qk + w.d_v) / 2.0
    return {"value": round(flops / dt / 1e12, 5), "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle", "seconds": round(dt, 2),
            "sample": f"{w.name}: query heads 0..{n_heads - 1} of {w.Hq} (KV heads "
                      f"0..{n_kv - 1}), all {w.N} rows, e4m3-decoded inputs in float64, "
                      f"O and LSE; TFLOP/s = the sample's causal FLOPs / oracle seconds"}


def copy_only(mib: int, reps: int = 3) -> int:
    """A plain device-to-device copy of `mib` MiB, for calibrating the HBM byte
    counters (FETCH_SIZE / WRITE_SIZE) against a known size."""
    import torch
    src = torch.ones(mib << 18, device="cuda:0", dtype=torch.float32)
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"bench: copied {mib} MiB x {reps}")
    return 0


def beyond_pages(ba, torch, w, xd, codes, ds, quant) -> dict:
    """Timings of the entry points past the pages' scope on the same workload: the
    Hadamard pre-step, chunked prefill (the last CHUNK queries over all keys) with the
    merge of two partial attentions, and the flash_attn_func wrapper's overhead."""
    out = {}
    # Hadamard rotation + quantisation of Q and K (HBM-bound: 2 fp32 reads + 1 code write)
    def quant_h():
        for n in "qk":
            ba.quantize_e4m3_hadamard(xd[n], codes[n], ds[n], per_head=w.fp8_per_head)
    t = time_events(quant_h, 10)
    hbytes = sum(xd[n].numel() * 9 for n in "qk")
    out["quantize_hadamard_qk_ms"] = round(t, 4)
    out["quantize_hadamard_qk_GBps"] = round(hbytes / t / 1e6, 1)
    quant()                                  # back to the plain codes
    # chunked prefill: queries N-CHUNK..N-1 over all N keys (key j visible to query i iff
    # j <= i + N - CHUNK), FP8 with LSE
    CHUNK = 4096
    N, dev = w.N, xd["q"].device
    off = N - CHUNK
    qc = codes["q"][:, off:]
    oc = torch.empty((w.B, CHUNK, w.Hq, w.d_v), device=dev, dtype=torch.bfloat16)
    lc = torch.empty((w.B, w.Hq, CHUNK), device=dev, dtype=torch.float32)
    pairs = CHUNK * (off + 1) + CHUNK * (CHUNK - 1) // 2
    fc = 2.0 * w.B * w.Hq * pairs * (w.d_qk + w.d_v)
    t = time_events(lambda: ba.attn_fwd_causal_offset_fp8(
        qc, codes["k"], codes["v"], ds["q"], ds["k"], ds["v"], oc, lc, q_offset=off,
        softmax_scale=w.softmax_scale, descale_per_head=int(w.fp8_per_head)), 10)
    out["chunk4k_of_32k_fp8_lse_ms"] = round(t, 4)
    out["chunk4k_of_32k_fp8_lse_tflops"] = round(fc / t / 1e9, 1)
    # merge of two partials of that chunk (HBM-bound: reads 2 O + 2 LSE, writes 1 + 1)
    ob = torch.empty_like(oc)
    lb = torch.empty_like(lc)
    om = torch.empty_like(oc)
    lm = torch.empty_like(lc)
    mbytes = 3 * (oc.numel() * 2 + lc.numel() * 4)
    ob.copy_(oc)
    lb.copy_(lc)
    t = time_events(lambda: ba.attn_merge_partials(oc, lc, ob, lb, om, lm), 20)
    out["merge_chunk4k_ms"] = round(t, 4)
    out["merge_chunk4k_GBps"] = round(mbytes / t / 1e6, 1)
    # flash_attn_func wrapper (allocates o and lse per call) against the entry point
    t_entry = time_events(lambda: ba.attn_fwd_causal_offset_fp8(
        qc, codes["k"], codes["v"], ds["q"], ds["k"], ds["v"], oc, lc, q_offset=off,
        softmax_scale=w.softmax_scale, descale_per_head=int(w.fp8_per_head)), 10)
    t_wrap = time_events(lambda: ba.flash_attn_func(
        qc, codes["k"], codes["v"], softmax_scale=w.softmax_scale, return_lse=True,
        q_descale=ds["q"], k_descale=ds["k"], v_descale=ds["v"]), 10)
    out["flash_attn_func_overhead_pct"] = round(100.0 * (t_wrap / t_entry - 1.0), 2)
    return out


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="gauss32k")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-extra", action="store_true")
    ap.add_argument("--cpu-heads", type=int, default=4)
    ap.add_argument("--profile-only", action="store_true",
                    help="run the step loop only (for rocprofv3), no JSON line")
    ap.add_argument("--profile-kernel",
                    choices=("step", "fp8", "bf16", "fp8_mla32k", "fp8_outliers_mistral16k"),
                    default="step",
                    help="with --profile-only: loop the step, the FP8 attention without the "
                         "LSE, the BF16 attention with the LSE, the FP8 attention with the LSE "
                         "on mla32k, or the exact-channel FP8 attention with the LSE on "
                         "mistral16k (the outlier path)")
    ap.add_argument("--copy-only", type=int, default=0, metavar="MIB",
                    help="run a plain device copy of MIB MiB (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on one GPU only: the attention kernels take one GPU's share "
              "of the work and no figure at several GPUs is produced; run with --gpus 1",
              file=sys.stderr)
        return 2
    if args.copy_only:
        return copy_only(args.copy_only)

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
    # the generated float32 buffers, hashed so that a run's inputs can be checked
    input_sha = {n: hashlib.sha256(x[n].tobytes()).hexdigest()[:16] for n in "qkv"}
    xd = {n: torch.from_numpy(x[n]).to(dev) for n in "qkv"}
    nds = lambda H: (H if w.fp8_per_head else 1)
    codes = {n: torch.empty(x[n].shape, device=dev, dtype=torch.uint8) for n in "qkv"}
    ds = {"q": torch.empty(nds(w.Hq), device=dev), "k": torch.empty(nds(w.Hkv), device=dev),
          "v": torch.empty(nds(w.Hkv), device=dev)}
    o = torch.empty((w.B, w.N, w.Hq, w.d_v), device=dev, dtype=torch.bfloat16)
    lse = torch.empty((w.B, w.Hq, w.N), device=dev, dtype=torch.float32)
    flops = workloads.causal_flops(w)

    def quant_separate():
        # K and V with their absmax scales, then Q with the scale that makes the FP8
        # softmax constant a power of two (given K's descales)
        for n in "kv":
            ba.quantize_e4m3(xd[n], codes[n], ds[n], per_head=w.fp8_per_head)
        ba.quantize_e4m3_q_pow2(xd["q"], codes["q"], ds["q"], ds["k"], w.softmax_scale,
                                per_head=w.fp8_per_head)

    def quant():
        # the same codes and descales in one call (four kernels instead of twelve)
        ba.quantize_e4m3_qkv(xd["q"], xd["k"], xd["v"], codes["q"], codes["k"], codes["v"],
                             ds["q"], ds["k"], ds["v"], per_head=w.fp8_per_head, q_pow2=True,
                             softmax_scale=w.softmax_scale)

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

    if args.profile_only and args.profile_kernel in ("fp8_mla32k", "fp8_outliers_mistral16k"):
        one = other_workload_loop(ba, torch, args.profile_kernel)
        for _ in range(args.warmup + args.steps):
            one()
        torch.cuda.synchronize()
        log(f"bench: profile-only {args.profile_kernel} run done")
        return 0
    if args.profile_only and args.profile_kernel != "step":
        if args.profile_kernel == "fp8":
            quant()
            one = lambda: attn_fp8(False)
        else:
            xb = {n: xd[n].to(torch.bfloat16) for n in "qkv"}
            one = lambda: ba.attn_fwd_causal_bf16(xb["q"], xb["k"], xb["v"], o, lse,
                                                  softmax_scale=w.softmax_scale)
        for _ in range(args.warmup + args.steps):
            one()
        torch.cuda.synchronize()
        log(f"bench: profile-only {args.profile_kernel} run done")
        return 0

    log(f"bench: warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev_attn.clear()
    log(f"bench: timing {args.steps} steps")
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
    attn_all = sorted(a.elapsed_time(b) for a, b in ev_attn)
    attn_ms = sum(attn_all) / len(attn_all)
    pct = lambda q: attn_all[min(len(attn_all) - 1, int(q * (len(attn_all) - 1) + 0.5))]
    value = flops / (ms_step * 1e-3) / 1e12
    achieved = flops / (attn_ms * 1e-3) / 1e12
    log(f"bench: step {ms_step:.3f} ms ({value:.1f} TFLOP/s); fp8 attention {attn_ms:.3f} ms "
        f"({achieved:.1f} TFLOP/s)")

    extra = {"fp8_attn_lse_ms": round(attn_ms, 4),
             "fp8_attn_lse_ms_p10_p50_p90": [round(pct(0.1), 4), round(pct(0.5), 4),
                                             round(pct(0.9), 4)]}
    if not args.no_extra:
        t = time_events(lambda: attn_fp8(False), 10)
        extra["fp8_attn_nolse_ms"] = round(t, 4)
        extra["fp8_attn_nolse_tflops"] = round(flops / t / 1e9, 1)
        # the same fast path writing the LSE of its rounded row sums (consistent with O)
        t = time_events(lambda: ba.attn_fwd_causal_offset_fp8_rounded_lse(
            codes["q"], codes["k"], codes["v"], ds["q"], ds["k"], ds["v"], o, lse, q_offset=0,
            softmax_scale=w.softmax_scale, descale_per_head=int(w.fp8_per_head)), 10)
        extra["fp8_attn_rounded_lse_tflops"] = round(flops / t / 1e9, 1)
        # the FP8 attention with the LSE on Q quantised with its plain absmax scale (the
        # softmax constant then takes one multiply-add per score)
        qa, da = torch.empty_like(codes["q"]), torch.empty_like(ds["q"])
        ba.quantize_e4m3(xd["q"], qa, da, per_head=w.fp8_per_head)
        t = time_events(lambda: ba.attn_fwd_causal_fp8(
            qa, codes["k"], codes["v"], da, ds["k"], ds["v"], o, lse,
            softmax_scale=w.softmax_scale, descale_per_head=int(w.fp8_per_head)), 10)
        extra["fp8_attn_lse_absmax_q_tflops"] = round(flops / t / 1e9, 1)
        del qa, da
        t = time_events(quant, 10)
        qbytes = sum(x[n].nbytes * 2 + x[n].size for n in "qkv")   # 2 reads + code write
        extra["quantize_qkv_ms"] = round(t, 4)
        extra["quantize_qkv_GBps"] = round(qbytes / t / 1e6, 1)
        t = time_events(quant_separate, 10)
        extra["quantize_qkv_separate_calls_ms"] = round(t, 4)
        extra.update(float32_q_lines(ba, w, xd, codes, ds, o, lse, flops))
        xb = {n: xd[n].to(torch.bfloat16) for n in "qkv"}
        for tag, L in (("bf16_attn_lse", lse), ("bf16_attn_nolse", None)):
            t = time_events(lambda: ba.attn_fwd_causal_bf16(xb["q"], xb["k"], xb["v"], o, L,
                                                            softmax_scale=w.softmax_scale), 10)
            extra[tag + "_tflops"] = round(flops / t / 1e9, 1)
        extra["bf16_attn_lse_pct_peak"] = round(
            100 * extra["bf16_attn_lse_tflops"] / PEAK_TFLOPS["bf16"], 2)
        # energy: the device's energy counter around back-to-back launches
        read, why = gpu_energy_reader()
        if read is None:
            extra["energy"] = {"unavailable": why}
        else:
            log("bench: energy runs")
            clock = gpu_clock_reader()
            extra["energy"] = {
                "fp8_attn_lse": energy_of(lambda: attn_fp8(True), flops, read, clock=clock),
                "fp8_attn_nolse": energy_of(lambda: attn_fp8(False), flops, read, clock=clock),
                "bf16_attn_lse": energy_of(
                    lambda: ba.attn_fwd_causal_bf16(xb["q"], xb["k"], xb["v"], o, lse,
                                                    softmax_scale=w.softmax_scale), flops, read,
                    clock=clock),
                "source": "amdsmi energy counter of the GPU (whole device), gauss32k"}
        del xb
        extra.update(beyond_pages(ba, torch, w, xd, codes, ds, quant))
        # kernel-only lines with sustained clock for every workload of the metric
        clock = gpu_clock_reader()
        extra["configs"] = {}
        for cname in ("mid_gqa", "mistral16k", "mla16k", "mla32k"):
            log(f"bench: kernel lines on {cname}")
            extra["configs"][cname] = config_lines(ba, torch, cname, clock)
        # the same lines on the headline workload (the exact-channel kernel's cost on
        # inputs without outlier channels, next to the plain kernel's)
        log("bench: kernel lines on gauss32k")
        extra["configs"]["gauss32k"] = config_lines(ba, torch, "gauss32k", clock)

    cpu = None
    if not args.no_cpu:
        log(f"bench: timing the CPU oracle on {args.cpu_heads} heads")
        cpu = cpu_baseline(w, x, args.cpu_heads)
        # a second sample on the MLA shape (two of its 16 heads), reported beside it
        import workloads
        wm = workloads.get("mla32k")
        log("bench: timing the CPU oracle on 2 heads of mla32k")
        extra["cpu_baseline_mla32k"] = cpu_baseline(wm, workloads.generate(wm), 2)

    # sustained shader clock: sampled from the device during the FP8-with-LSE energy loop
    sclk = (extra.get("energy", {}).get("fp8_attn_lse") or {}).get("sclk_mhz")
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
        "vs_baseline": None,
        "dtype": "fp8_e4m3",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "N": w.N,
                   "d_qk": w.d_qk, "d_v": w.d_v, "inputs": "iid N(0,1) float32 in HBM",
                   "seed": w.seed, "numpy": np.__version__, "inputs_sha256": input_sha,
                   "step": "quantize_e4m3_qkv (k, v absmax, q power-of-two scale), per "
                            "tensor, + attn_fwd_causal_fp8 (O + LSE)"},
        "pct_peak": round(100 * value / PEAK_TFLOPS["fp8"], 2),
        "roofline": {"bound": "mfma", "kernel": "attn_fwd_kernel<fp8, d128> (with LSE)",
                     "achieved": round(achieved, 2), "peak": PEAK_TFLOPS["fp8"],
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_TFLOPS["fp8"], 4),
                     "traffic": traffic_from_profile("attn_fwd_fp8_d128_lse_gauss32k")},
        "sclk_mhz": sclk,
        "frac_of_clock_adjusted_peak": (round(achieved / (PEAK_TFLOPS["fp8"] * sclk / 2400.0), 4)
                                        if sclk else None),
        "cpu_baseline": cpu,
        "context": {"pages_fp8_d128_32k_tflops": PAGES_FP8_D128_32K,
                    "note": "the pages' MI355X kernel figure; B, H and LSE handling unstated"},
        "extra": extra,
    }
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
