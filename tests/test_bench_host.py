"""Host-side logic of bench.py, checked on the CPU: the one-GPU refusal, the
kernel-source hash that decides whether the committed HBM counters still
apply, the lookup of those counters, and the routing step's byte count."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_source_hash_ignores_comments_and_spacing(tmp_path, monkeypatch):
    a = tmp_path / "a.hip"
    b = tmp_path / "b.hip"
    c = tmp_path / "c.hip"
    a.write_text("int f(int x) {  // doubles\n  return 2 * x;\n}\n")
    b.write_text("/* a comment */ int f(int x){return 2*x;}   // another\n")
    c.write_text("int f(int x) { return 3 * x; }\n")
    monkeypatch.setattr(bench, "KERNEL_SOURCES", [str(a)])
    ha = bench.kernel_source_hash()
    monkeypatch.setattr(bench, "KERNEL_SOURCES", [str(b)])
    hb = bench.kernel_source_hash()
    monkeypatch.setattr(bench, "KERNEL_SOURCES", [str(c)])
    hc = bench.kernel_source_hash()
    assert ha == hb and ha != hc
    assert len(ha) == 16 and int(ha, 16) >= 0


def test_source_hash_of_the_kernel_is_stable():
    assert bench.kernel_source_hash() == bench.kernel_source_hash()


def test_traffic_only_while_the_kernel_is_unchanged(tmp_path, monkeypatch):
    counters = tmp_path / "counters.txt"
    counters.write_text("# header: with a colon\n"
                        "kernel_source_sha256_16: 0123456789abcdef\n"
                        "hbm_bytes_per_launch_calibrated: 12345\n")
    monkeypatch.setattr(bench, "COUNTERS", str(counters))
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "0123456789abcdef")
    assert bench.measured_traffic("prefill") == 12345.0
    assert bench.measured_traffic("decode") is None          # counters are for prefill only
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "fedcba9876543210")
    assert bench.measured_traffic("prefill") is None          # the kernel changed since
    monkeypatch.setattr(bench, "COUNTERS", str(tmp_path / "missing.txt"))
    assert bench.measured_traffic("prefill") is None


def test_committed_counter_file_parses():
    """The committed summary carries the three keys bench.py reads."""
    vals = {}
    for line in open(bench.COUNTERS):
        if ":" in line and not line.startswith("#"):
            key, val = line.split(":", 1)
            vals[key.strip()] = val.strip()
    assert len(vals["kernel_source_sha256_16"]) == 16
    assert float(vals["hbm_bytes_per_launch_calibrated"]) == pytest.approx(
        float(vals["hbm_fetch_bytes_per_launch_calibrated"])
        + float(vals["hbm_write_bytes_per_launch_calibrated"]), rel=1e-9)


def test_routing_bytes():
    T, H, N, k = 16, 256, 128, 4
    common = N * 4 + T * N * 4 + T * k * 8          # bias in; scores, (index, gate) out
    assert bench.route_bytes_of(T, H, N, k, False) == common + T * H * 2 + N * H * 2
    xq = T * H + T * (H // 128) * 4                 # x codes and scales: written, read back
    assert bench.route_bytes_of(T, H, N, k, True) == (common + T * H * 2 + 2 * xq + N * H
                                                      + (N // 128) * (H // 128) * 4)
    # at the routing workload's shape the bf16 router moves about 256 MB
    assert bench.route_bytes_of(16384, 7168, 256, 8, False) == 256377856
