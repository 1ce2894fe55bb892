"""bench.py's contract on the host: one GPU only, and the HBM traffic it
reports comes from the committed counter summary, scaled by the copy-kernel
factors, only while the kernel sources are the ones the counters were taken
on."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""  # no JSON line


def _summary():
    kv = {}
    with open(os.path.join(ROOT, bench.TRAFFIC_SUMMARY)) as f:
        for line in f:
            if "=" in line and not line.lstrip().startswith("#"):
                k, v = line.split("=", 1)
                kv[k.strip()] = v.strip()
    return kv


def test_traffic_summary_is_self_consistent():
    kv = _summary()
    probe = float(kv["copy_probe_bytes"])
    fs = probe / (float(kv["copy_fetch_kib_per_dispatch"]) * 1024)
    ws = probe / (float(kv["copy_write_kib_per_dispatch"]) * 1024)
    assert fs == pytest.approx(float(kv["fetch_scale"]), rel=1e-5)
    assert ws == pytest.approx(float(kv["write_scale"]), rel=1e-5)
    t = float(kv["fetch_kib_per_dispatch"]) * 1024 * fs + float(kv["write_kib_per_dispatch"]) * 1024 * ws
    assert t == pytest.approx(float(kv["traffic_bytes_per_launch"]), rel=1e-5)
    # at least the algorithmic bytes of one launch (codes, scales, means, fp32 output)
    assert t >= 2.7e9


def test_traffic_only_for_the_same_sources_and_workload(monkeypatch):
    kv = _summary()
    if kv.get("source_sha256") == bench.kernel_source_hash():
        assert bench.measured_traffic(kv["workload"]) == float(kv["traffic_bytes_per_launch"])
    assert bench.measured_traffic("tiny") is None
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "0" * 64)
    assert bench.measured_traffic(kv["workload"]) is None


def test_skip_fractions_on_byte_dumps():
    import torch
    nb = 3
    full = torch.ones((256, nb * 128), dtype=torch.uint8)
    skip = full.clone()
    skip[0:32, 128:256] = 0      # wave 0 rejects block 1 in every row
    skip[32:40, 256:384] = 0     # 8 rows of wave 1 reject block 2
    row, wave = bench.skip_fractions(full, skip, nb)
    assert row == pytest.approx((32 + 8) / (256 * nb), rel=1e-6)
    assert wave == pytest.approx(1 / (8 * nb), rel=1e-6)
