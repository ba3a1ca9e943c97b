"""Host-side logic of bench.py (CPU only, no GPU): the one-GPU rule, the kernel-source
hash that ties profiles/traffic.json to the kernel it was measured on, the traffic
lookup, and the CPU-oracle baseline record on a small workload."""
import json
import os
import subprocess
import sys

import bench
import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       cwd=ROOT, capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "gpus 1" in (r.stdout + r.stderr)
    assert not r.stdout.strip().startswith("{")      # no JSON line


def test_kernel_source_hash_is_stable_and_covers_the_kernel_files():
    a, b = bench.kernel_source_sha(), bench.kernel_source_sha()
    assert a == b and len(a) == 16
    for name in bench.KERNEL_SOURCES:
        assert os.path.exists(os.path.join(ROOT, "bf16_causal_prefill_amd", "csrc", name))


def test_traffic_lookup_follows_the_source_hash(tmp_path, monkeypatch):
    (tmp_path / "profiles").mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_source_sha", lambda: "0123456789abcdef")
    path = tmp_path / "profiles" / "traffic.json"
    path.write_text(json.dumps({"k": {"source_sha": "0123456789abcdef",
                                      "hbm_bytes_per_launch": 123}}))
    assert bench.traffic_from_profile("k") == 123
    assert bench.traffic_from_profile("missing") is None
    path.write_text(json.dumps({"k": {"source_sha": "fedcba9876543210",
                                      "hbm_bytes_per_launch": 123}}))
    assert bench.traffic_from_profile("k") is None      # measured on other sources


def test_cpu_baseline_record():
    w = workloads.get("tiny").with_(N=64)
    rec = bench.cpu_baseline(w, workloads.generate(w), 2)
    assert rec["kind"] == "oracle" and rec["unit"] == "TFLOP/s"
    assert rec["value"] > 0 and rec["cores"] >= 1 and rec["seconds"] >= 0
    assert "query heads 0..1" in rec["sample"]
