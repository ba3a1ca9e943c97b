"""Phase timers of the attention kernels on the full workloads (needs one MI355X).

Loads the measurement build libattn_phase_timers.so (built by
`python -m bf16_causal_prefill_amd.build --phase-timers`, or by __graft_entry__.build()),
in which every wave reads the shader clock around the two phases of each key tile of
the two-group schedule (include/attn_phase_timers.h), and writes, per workload, the
mean cycles per key tile of the matrix phase, the softmax phase and the whole period,
per wave group, to OUTDIR/phase_timers_<workload>.txt (then copied into profiles/).

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

RECORD_BLOCKS = 256
WAVES, WORDS = 8, 4           # include/attn_phase_timers.h


def main() -> int:
    import torch

    import bf16_causal_prefill_amd as ba
    import workloads

    out_dir = sys.argv[1] if len(sys.argv) > 1 else os.path.join(ROOT, "gpurun_out", "profiles")
    names = sys.argv[2:] or ["gauss32k", "mla32k", "mistral16k"]
    os.makedirs(out_dir, exist_ok=True)
    ba.load_library(ba.PHASE_TIMERS_LIB_PATH)
    dev = "cuda:0"
    buf = torch.zeros(RECORD_BLOCKS * WAVES * WORDS, dtype=torch.int64, device=dev)
    command = "python profile_phases.py " + " ".join(sys.argv[1:])

    for name in names:
        w = workloads.get(name)
        print(f"phase timers: {name} (B={w.B} Hq={w.Hq} Hkv={w.Hkv} N={w.N} "
              f"d={w.d_qk}/{w.d_v})", flush=True)
        x = workloads.generate(w)
        xd = {n: torch.from_numpy(x[n]).to(dev) for n in "qkv"}
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
                 f"# the first {RECORD_BLOCKS} workgroups of one launch after ~1 s of back-to-back "
                 "calls; waves with >= 8 counted tiles; group A = waves 0-3 (matrix phase first)",
                 "# busy = cycles from a phase's start to its barrier; wait = period - busy(matrix) "
                 "- busy(softmax), time spent at the two barriers",
                 "",
                 f"{'kernel':52s} {'grp':>3s} {'waves':>5s} {'period':>7s} {'matrix':>7s} "
                 f"{'softmax':>7s} {'wait':>6s}"]
        for title, fn in kernels:
            t0 = time.time()
            while time.time() - t0 < 1.0:
                for _ in range(5):
                    fn()
                torch.cuda.synchronize()
            buf.zero_()
            torch.cuda.synchronize()
            ba.attn_phase_timers_set(buf)
            fn()
            torch.cuda.synchronize()
            ba.attn_phase_timers_set(None)
            rec = buf.view(RECORD_BLOCKS, WAVES, WORDS).cpu().numpy()
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
        path = os.path.join(out_dir, f"phase_timers_{name}.txt")
        with open(path, "w") as f:
            f.write("\n".join(lines) + "\n")
        print(f"phase timers written to {path}", flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
