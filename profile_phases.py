"""Phase timers of the attention kernels on the full workloads (needs one MI355X).

Loads the measurement build libattn_phase_timers.so (built by
`python -m bf16_causal_prefill_amd.build --phase-timers`, or by __graft_entry__.build()),
in which every wave reads the shader clock around the two phases of each key tile of
the two-group schedule (include/attn_phase_timers.h), and writes, per workload, the
mean cycles per key tile of the matrix phase, the softmax phase and the whole period,
per wave group, to OUTDIR/phase_timers_<workload>.txt (then copied into profiles/).
The same records carry the device's real-time counter at each wave's start, loop entry,
loop exit and end (its stores issued) and the wave's CU: the file's second table gives, per
kernel, the prologue and the epilogue, the time per key tile, and the gap between one
workgroup's end and the next one's start on the same CU, over every workgroup of the launch;
a third table gives the balance over the 8 XCDs (busy time per CU of each, odd over even)
and the gaps per shader engine.

Usage: python profile_phases.py [OUTDIR] [workload ...]
(default OUTDIR gpurun_out/profiles; workloads gauss32k mla32k mistral16k)

Each kernel runs back to back for about a second first (so the clock has settled),
then once with the timers set; the first 256 workgroups of that launch (the heaviest
causal tiles, launched first, so every one walks many tiles) are summarised, waves with
at least 8 counted tiles only.  The clock reads sit between scheduling barriers, so the
timed build's instruction order differs slightly from the product's; the figures show
which phase sets the period, not the product's speed.
"""
from __future__ import annotations

import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PHASE_BLOCKS = 256             # workgroups summarised in the phase table
WAVES, WORDS = 8, 10           # include/attn_phase_timers.h
BM = 256                       # queries per workgroup (8 waves of 32)
REALTIME_MHZ = 100.0           # rate of the device's real-time counter (checked per launch)


def timeline(rec, event_ms):
    """Per-kernel figures from the real-time words of every workgroup's records: prologue
    (waves 0-3, which enter the loop first) and epilogue in µs, µs per key tile (the loop
    of group A's waves over its tiles + 1 matrix phases), the gap between consecutive
    workgroups on one CU, and the counter rate implied by the launch's span against its
    event-timed duration."""
    import numpy as np
    used = rec[:, 0, 4] != 0
    r = rec[used].astype(np.int64)
    us = lambda ticks: ticks / REALTIME_MHZ
    pro = us(r[:, 0:4, 5] - r[:, 0:4, 4]).mean()
    epi = us(r[:, :, 7] - r[:, :, 6]).mean()
    tile = (us(r[:, 0:4, 6] - r[:, 0:4, 5]) / (r[:, 0:4, 8] + 1)).mean()
    start, end = r[:, :, 4].min(axis=1), r[:, :, 7].max(axis=1)
    cu = ((r[:, 0, 9] >> 8) & 0xFF) | (((r[:, 0, 9] >> 32) & 0xFF) << 8)
    gaps, per_cu = [], []
    for c in np.unique(cu):
        idx = np.where(cu == c)[0]
        order = idx[np.argsort(start[idx])]
        per_cu.append(len(order))
        gaps += list(us(start[order[1:]] - end[order[:-1]]))
    gaps = np.array(gaps) if gaps else np.zeros(1)
    mhz = (end.max() - start.min()) / (event_ms * 1e3)
    # balance: busy µs per CU of each XCD (from XCC_ID), and the mean gap per shader engine
    # (HW_ID bits 13-15) over all XCDs
    xcc = (r[:, 0, 9] >> 32) & 0xF
    se = (r[:, 0, 9] >> 13) & 0x7
    busy = [float(us(end - start)[xcc == x].sum()) / max(1, len(np.unique(cu[xcc == x])))
            for x in range(8)]
    se_gap = []
    for e in range(4):
        g = []
        for c in np.unique(cu[se == e]):
            idx = np.where(cu == c)[0]
            order = idx[np.argsort(start[idx])]
            g += list(us(start[order[1:]] - end[order[:-1]]))
        se_gap.append(float(np.mean(g)) if g else 0.0)
    even, odd = np.mean(busy[0::2]), np.mean(busy[1::2])
    return {"workgroups": int(used.sum()), "cus": len(per_cu), "prologue": pro, "epilogue": epi,
            "tile": tile, "gap_mean": float(gaps.mean()), "gap_median": float(np.median(gaps)),
            "pairs": int(len(gaps)), "span_over_event_mhz": float(mhz),
            "xcd_busy": busy, "odd_over_even": float(odd / even) if even > 0 else 0.0,
            "span_over_mean_xcd": float(us(end.max() - start.min()) / np.mean(busy)),
            "se_gap": se_gap}


def main() -> int:
    import torch

    import bf16_causal_prefill_amd as ba
    import workloads

    out_dir = sys.argv[1] if len(sys.argv) > 1 else os.path.join(ROOT, "gpurun_out", "profiles")
    names = sys.argv[2:] or ["gauss32k", "mla32k", "mistral16k"]
    os.makedirs(out_dir, exist_ok=True)
    ba.load_library(ba.PHASE_TIMERS_LIB_PATH)
    dev = "cuda:0"
    command = "python profile_phases.py " + " ".join(sys.argv[1:])

    for name in names:
        w = workloads.get(name)
        print(f"phase timers: {name} (B={w.B} Hq={w.Hq} Hkv={w.Hkv} N={w.N} "
              f"d={w.d_qk}/{w.d_v})", flush=True)
        x = workloads.generate(w)
        xd = {n: torch.from_numpy(x[n]).to(dev) for n in "qkv"}
        blocks = -(-w.N // BM) * w.B * w.Hq     # the launch's workgroups, all recorded
        buf = torch.zeros(blocks * WAVES * WORDS, dtype=torch.int64, device=dev)
        ph = w.fp8_per_head
        nds = lambda H: (H if ph else 1)
        codes = {n: torch.empty(x[n].shape, device=dev, dtype=torch.uint8) for n in "qkv"}
        ds = {"q": torch.empty(nds(w.Hq), device=dev), "k": torch.empty(nds(w.Hkv), device=dev),
              "v": torch.empty(nds(w.Hkv), device=dev)}
        for n in "kv":
            ba.quantize_e4m3(xd[n], codes[n], ds[n], per_head=ph)
        q_abs = torch.empty_like(codes["q"])
        dq_abs = torch.empty_like(ds["q"])
        ba.quantize_e4m3(xd["q"], q_abs, dq_abs, per_head=ph)
        ba.quantize_e4m3_q_pow2(xd["q"], codes["q"], ds["q"], ds["k"], w.softmax_scale, per_head=ph)
        bf = {n: xd[n].to(torch.bfloat16) for n in "qkv"}
        o = torch.empty((w.B, w.N, w.Hq, w.d_v), device=dev, dtype=torch.bfloat16)
        lse = torch.empty((w.B, w.Hq, w.N), device=dev, dtype=torch.float32)
        s, iph = w.softmax_scale, int(ph)
        fp8 = lambda qc, qd, L: (lambda: ba.attn_fwd_causal_fp8(
            qc, codes["k"], codes["v"], qd, ds["k"], ds["v"], o, L, softmax_scale=s,
            descale_per_head=iph))
        kernels = [
            ("FP8 with LSE, power-of-two Q scale (exact P)", fp8(codes["q"], ds["q"], lse)),
            ("FP8 with LSE, absmax Q scale (exact P)", fp8(q_abs, dq_abs, lse)),
            ("FP8 without LSE (Lean P)", fp8(codes["q"], ds["q"], None)),
            ("BF16 with LSE", lambda: ba.attn_fwd_causal_bf16(bf["q"], bf["k"], bf["v"], o, lse,
                                                              softmax_scale=s)),
        ]
        if w.d_qk == 128 and w.recipe == "mistral":
            T = ba.OUTLIER_CHANNELS
            qo, ko = torch.empty_like(codes["q"]), torch.empty_like(codes["k"])
            qx = torch.empty((w.B, w.N, w.Hq, T), device=dev, dtype=torch.bfloat16)
            kx = torch.empty((w.B, w.N, w.Hkv, T), device=dev, dtype=torch.bfloat16)
            dqo, dko = torch.empty_like(ds["q"]), torch.empty_like(ds["k"])
            perm = torch.empty((w.Hkv, w.d_qk), device=dev, dtype=torch.uint8)
            ba.quantize_e4m3_qk_outliers(xd["q"], xd["k"], qo, ko, qx, kx, dqo, dko, perm, ph,
                                         q_pow2=True, softmax_scale=s)
            ex = lambda L: (lambda: ba.attn_fwd_causal_fp8_outliers(
                qo, ko, codes["v"], qx, kx, dqo, dko, ds["v"], o, L, softmax_scale=s,
                descale_per_head=iph))
            kernels += [("FP8 exact channels with LSE, power-of-two Q scale", ex(lse)),
                        ("FP8 exact channels without LSE", ex(None))]

        lines = [f"# phase timers per 128-key tile (64 for BF16) and wave, shader cycles: {name} "
                 f"(B={w.B} Hq={w.Hq} Hkv={w.Hkv} N={w.N} d={w.d_qk}/{w.d_v})",
                 f"# command: {command}",
                 "# build: libattn_phase_timers.so (python -m bf16_causal_prefill_amd.build "
                 "--phase-timers); record layout in include/attn_phase_timers.h",
                 f"# the first {PHASE_BLOCKS} workgroups of one launch after ~1 s of back-to-back "
                 "calls; waves with >= 8 counted tiles; group A = waves 0-3 (matrix phase first)",
                 "# busy = cycles from a phase's start to its barrier; wait = period - busy(matrix) "
                 "- busy(softmax), time spent at the two barriers",
                 "",
                 f"{'kernel':52s} {'grp':>3s} {'waves':>5s} {'period':>7s} {'matrix':>7s} "
                 f"{'softmax':>7s} {'wait':>6s}"]
        tl_rows, bal_rows = [], []
        for title, fn in kernels:
            t0 = time.time()
            while time.time() - t0 < 1.0:
                for _ in range(5):
                    fn()
                torch.cuda.synchronize()
            buf.zero_()
            torch.cuda.synchronize()
            ba.attn_phase_timers_set(buf)
            ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            ev0.record()
            fn()
            ev1.record()
            torch.cuda.synchronize()
            ba.attn_phase_timers_set(None)
            rec_all = buf.view(blocks, WAVES, WORDS).cpu().numpy()
            tl = timeline(rec_all, ev0.elapsed_time(ev1))
            tl_rows.append(f"{title:52s} {tl['workgroups']:5d} {tl['cus']:4d} {tl['prologue']:8.2f} "
                           f"{tl['epilogue']:8.2f} {tl['tile']:6.3f} {tl['gap_mean']:8.2f} "
                           f"{tl['gap_median']:8.2f} {tl['span_over_event_mhz']:7.1f}")
            print("  " + tl_rows[-1], flush=True)
            bal_rows.append(f"{title:52s} " + " ".join(f"{b:6.0f}" for b in tl["xcd_busy"]) +
                            f" {tl['odd_over_even']:7.4f} {tl['span_over_mean_xcd']:7.4f}  " +
                            " ".join(f"{g:5.2f}" for g in tl["se_gap"]))
            rec = rec_all[:PHASE_BLOCKS]
            for grp, waves in (("A", range(0, 4)), ("B", range(4, 8))):
                r = rec[:, list(waves), :].reshape(-1, WORDS)
                r = r[r[:, 0] >= 8]
                if len(r) == 0:
                    continue
                n = r[:, 0].astype(float)
                mb, vb, per = (float((r[:, j] / n).mean()) for j in (1, 2, 3))
                lines.append(f"{title:52s} {grp:>3s} {len(r):5d} {per:7.0f} {mb:7.0f} {vb:7.0f} "
                             f"{per - mb - vb:6.0f}")
            print("  " + lines[-1], flush=True)
        lines += ["",
                  f"# per-workgroup timeline from the real-time words, every workgroup of the "
                  f"launch, µs at {REALTIME_MHZ:.0f} MHz: prologue = loop entry - start (waves "
                  "0-3); epilogue = O/LSE stores issued - loop exit (all waves); tile = "
                  "loop time / (key tiles + 1) (waves 0-3); gap = next workgroup's first wave "
                  "start - this one's last wave end on the same CU; rate = the launch's real-time "
                  "span over its event-timed duration (MHz, a check of the counter's rate)",
                  "",
                  f"{'kernel':52s} {'wgs':>5s} {'cus':>4s} {'prologue':>8s} {'epilogue':>8s} "
                  f"{'tile':>6s} {'gap':>8s} {'gap_med':>8s} {'rate':>7s}"] + tl_rows
        lines += ["",
                  "# balance over the dies and shader engines, same launches: busy µs per CU of each "
                  "XCD (XCC_ID 0-7), the odd XCDs' mean over the even ones', the launch's span over "
                  "the mean XCD's busy time, and the mean gap (µs) between workgroups on one CU per "
                  "shader engine 0-3 (HW_ID bits 13-15)",
                  "",
                  f"{'kernel':52s} " + " ".join(f"{'xcd' + str(x):>6s}" for x in range(8)) +
                  f" {'odd/ev':>7s} {'span/m':>7s}  " + " ".join(f"{'se' + str(e):>5s}" for e in range(4))] + bal_rows
        path = os.path.join(out_dir, f"phase_timers_{name}.txt")
        with open(path, "w") as f:
            f.write("\n".join(lines) + "\n")
        print(f"phase timers written to {path}", flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
