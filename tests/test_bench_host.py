"""Host logic of bench.py that runs without a GPU: the one-GPU guard and the rule that the
measured HBM traffic is reported only for the kernel sources it was counted on."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode != 0
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in msg["error"]


def test_traffic_is_read_for_the_counted_sources_only(tmp_path, monkeypatch):
    sha = bench.kernel_source_sha()
    f = tmp_path / "traffic.txt"
    f.write_text(f"traffic_bytes_per_launch: 73231273\nsource_sha256: {sha}\n")
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.measured_traffic(1 << 20, 8) == 73231273
    # another workload than the one counted
    assert bench.measured_traffic(1 << 21, 8) is None
    assert bench.measured_traffic(1 << 20, 4) is None
    # counters taken on other sources
    f.write_text("traffic_bytes_per_launch: 73231273\nsource_sha256: " + "0" * 64 + "\n")
    assert bench.measured_traffic(1 << 20, 8) is None


def test_source_hash_ignores_comments_but_not_code(tmp_path, monkeypatch):
    a = tmp_path / "k.h"
    a.write_text("int x = 1;  // one\n\n// note\nint y = 2;\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "KERNEL_SOURCES", ["k.h"])
    h0 = bench.kernel_source_sha()
    a.write_text("int x = 1;  // first\n// other note\n\nint y = 2;\n")
    assert bench.kernel_source_sha() == h0
    a.write_text("int x = 1;\nint y = 3;\n")
    assert bench.kernel_source_sha() != h0

