"""The workgroup -> (batch, query head, query tile) map of the attention kernels, checked on
the host: tests/tile_map_host.cpp includes the kernel header, built host-only (the map and
the launcher's schedule are host-callable), and walks every workgroup of 100 launches
(20 shapes: square and offset, GQA ratios 1-8, B up to 16, N from 1 to 50000; FP8 in the
three LSE modes and BF16 in two), checking that every tile is computed exactly once, that
each XCD runs only its pair's KV groups at the places the exchange plan allows, and that
the planned shift of work from the odd to the even XCDs lands within the plan's tolerance."""
import os
import subprocess

import pytest

from bf16_causal_prefill_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_tile_map_on_the_host(tmp_path):
    try:
        hipcc = build._hipcc()
    except RuntimeError:
        pytest.skip("hipcc not found")
    exe = tmp_path / "tile_map_host"
    cmd = [hipcc, "-std=c++17", "-O1", "--offload-host-only", "-x", "hip",
           "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "tile_map_host.cpp"),
           "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-3000:]
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    print(r.stdout[-2000:])
    assert r.returncode == 0, r.stdout[-3000:]
    last = r.stdout.strip().splitlines()[-1].split()
    counts = dict(zip(last[0::2], map(int, last[1::2])))
    assert counts["cases"] == 100 and counts["failures"] == 0
    assert counts["exchange"] > 0 and counts["rotate"] > 0   # both paths exercised
