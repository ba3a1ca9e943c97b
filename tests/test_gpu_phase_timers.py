"""The phase-timer measurement build (libattn_phase_timers.so) on the GPU: profile_phases.py
runs in a child process (the package loads one library per process) on the 4K workload
and writes a summary whose figures must be complete and consistent for every kernel
variant and both wave groups: counted tiles present, every phase a positive number of
cycles, and the period no shorter than the two phases' busy time; and, from the
real-time words, every workgroup of the launch recorded, on as many CUs as the device
has (one workgroup per CU at a time, so no negative gaps), positive prologue, epilogue
and tile times, and the counter's rate no higher than the launch's event-timed span allows;
and the balance table: every XCD busy, the odd/even ratio within 20%, the span no shorter
than the mean XCD's busy time, non-negative gaps on every shader engine."""
import os
import subprocess
import sys

import pytest

import bf16_causal_prefill_amd as ba

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

KERNELS = ["FP8 with LSE, power-of-two Q scale (exact P)", "FP8 with LSE, absmax Q scale (exact P)",
           "FP8 without LSE (Lean P)", "BF16 with LSE"]


@pytest.mark.skipif(not os.path.exists(ba.PHASE_TIMERS_LIB_PATH),
                    reason="libattn_phase_timers.so not built (build.py --phase-timers)")
def test_phase_timer_summary(tmp_path):
    r = subprocess.run([sys.executable, "-u", os.path.join(ROOT, "profile_phases.py"),
                        str(tmp_path), "mid_gqa"], cwd=ROOT, capture_output=True, text=True,
                       timeout=240)
    print(r.stdout[-3000:])
    assert r.returncode == 0, r.stderr[-3000:]
    text = (tmp_path / "phase_timers_mid_gqa.txt").read_text()
    phases, rest = text.split("# per-workgroup timeline")
    timeline, balance = rest.split("# balance over")
    rows = {}
    for line in phases.splitlines():
        if line.startswith("#") or not line.strip() or line.startswith("kernel"):
            continue
        name, rest = line[:52].strip(), line[52:].split()
        grp, waves, period, matrix, softmax, wait = rest[0], *map(float, rest[1:])
        rows[(name, grp)] = (waves, period, matrix, softmax, wait)
    tl = {}
    for line in timeline.splitlines()[1:]:
        if line.startswith("#") or not line.strip() or line.startswith("kernel"):
            continue
        tl[line[:52].strip()] = list(map(float, line[52:].split()))
    grid = 4096 // 256 * 32          # mid_gqa: 16 query tiles x 32 heads
    for k in KERNELS:
        wgs, cus, pro, epi, tile, gap, gap_med, rate = tl[k]
        assert wgs == grid, (k, tl[k])
        assert 128 <= cus <= 256, (k, tl[k])
        assert pro > 0 and epi > 0 and tile > 0, (k, tl[k])
        assert gap >= 0 and gap_med >= 0, (k, tl[k])
        # the event-timed duration includes the launch's own latency (tens of µs at times,
        # against a 4K launch's ~75 µs), so the span's rate reads below the counter's
        # 100 MHz, never above it; the floor only catches a counter off by an order of
        # magnitude (the 16K and 32K launches read 98-99.7 MHz)
        assert 20 <= rate <= 102, (k, tl[k])
    bal = {}
    for line in balance.splitlines()[1:]:
        if line.startswith("#") or not line.strip() or line.startswith("kernel"):
            continue
        bal[line[:52].strip()] = list(map(float, line[52:].split()))
    for k in KERNELS:
        busy, ratio, span_m, se_gap = bal[k][:8], bal[k][8], bal[k][9], bal[k][10:]
        assert len(se_gap) == 4 and all(b > 0 for b in busy), (k, bal[k])
        # the XCDs differ by a few percent; the launch cannot end before its mean XCD
        assert 0.8 < ratio < 1.25 and span_m >= 0.99, (k, bal[k])
        assert all(g >= 0 for g in se_gap), (k, bal[k])
    for k in KERNELS:
        for grp in "AB":
            waves, period, matrix, softmax, wait = rows[(k, grp)]
            assert waves > 0, (k, grp)
            assert matrix > 0 and softmax > 0, (k, grp, rows[(k, grp)])
            assert period >= matrix + softmax - 1, (k, grp, rows[(k, grp)])
            # a key tile takes at least the 16 matrix instructions' 1024 cycles per group
            assert period >= 1024, (k, grp, rows[(k, grp)])
