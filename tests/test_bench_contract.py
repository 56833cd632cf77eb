"""CPU checks of the benchmark harness (no GPU work runs here)."""
import os
import subprocess
import sys

import bench_counters

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode != 0
    assert "single GPU" in r.stderr


def test_traffic_summary_is_read_only_for_the_current_kernel(tmp_path):
    sha = bench_counters.kernel_source_sha()
    body = ("# header\n"
            f"kernel_source_sha256: {sha}\n"
            "copy_calibration: bytes=1 fetch_kib=1 write_kib=1 fetch_scale=2 write_scale=1\n"
            "launch q+k+v: dispatches=7 fetch_kib=1.00 write_kib=1.00 traffic_bytes=123\n"
            "launch o: dispatches=7 fetch_kib=1.00 write_kib=1.00 traffic_bytes=45\n")
    p = tmp_path / "t.txt"
    p.write_text(body)
    assert bench_counters.read_traffic(str(p)) == {"q+k+v": 123.0, "o": 45.0}
    p.write_text(body.replace(sha, "0" * 64))
    assert bench_counters.read_traffic(str(p)) is None
    assert bench_counters.read_traffic(str(tmp_path / "missing.txt")) is None


def test_launches_are_split_by_dispatch_order():
    per = bench_counters._by_launch(list(range(8)), "test")
    assert per == {"q+k+v": [0, 4], "o": [1, 5], "gate+up": [2, 6], "down": [3, 7]}
