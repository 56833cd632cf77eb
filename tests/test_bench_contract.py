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
    # one eager warmup step, the graph of two steps replayed twice (16 dispatches), then the roofline leg:
    # one eager warmup launch and its graph of two launches replayed twice
    per, tail = bench_counters._by_launch(list(range(20 + 5)), 1, 2, "test")
    assert per == {"q+k+v": [12, 16], "o": [13, 17], "gate+up": [14, 18], "down": [15, 19]}
    assert tail == [23, 24]
    try:
        bench_counters._by_launch(list(range(20 + 4)), 1, 2, "test")
    except SystemExit:
        pass
    else:
        raise AssertionError("a trace without the roofline leg must be rejected")


def test_workload_passes_follow_decode_order():
    import bench_configs
    import workloads as W
    # 9B layer: q+k+v | o | gate+up | down
    assert bench_configs.launch_groups(W.config(4).matrices) == [[0, 1, 2], [3], [4, 5], [6]]
    # 131M set: no gate, so up and down launch alone; 12 layers x 4 launches
    g = bench_configs.launch_groups(W.config(2).matrices)
    assert len(g) == 48 and g[:4] == [[0, 1, 2], [3], [4], [5]]
    # every matrix exactly once, in order
    for cid in W.ALL_CONFIGS:
        flat = [i for grp in bench_configs.launch_groups(W.config(cid).matrices) for i in grp]
        assert flat == list(range(len(W.config(cid).matrices)))


def test_kernel_summary_groups_dispatches_by_kernel(tmp_path):
    cols = ["Kind", "Kernel_Name", "Start_Timestamp", "End_Timestamp", "LDS_Block_Size", "Scratch_Size",
            "VGPR_Count", "SGPR_Count", "Grid_Size_X", "Grid_Size_Y"]
    rows = [["KERNEL_DISPATCH", "gemv_tiles<true>(Batch)", "1000", "3000", "28160", "0", "48", "112", "256", "1"],
            ["KERNEL_DISPATCH", "gemv_tiles<true>(Batch)", "5000", "9000", "28160", "0", "48", "112", "256", "1"],
            ["KERNEL_DISPATCH", "copyBuffer", "0", "100", "0", "0", "8", "32", "1", "1"],
            ["KERNEL_DISPATCH", "gemm_frag<1u, 8u, true>(GemmArgs)", "0", "10000", "35328", "0", "56", "80", "256", "1"]]
    p = tmp_path / "kt.csv"
    p.write_text("\n".join(",".join(f'"{v}"' for v in r) for r in [cols] + rows) + "\n")

    class A:
        csv = str(p)
        title = "t"
        command = "c"
    text = bench_counters.kernels_summary(A)
    assert "copyBuffer" not in text
    assert "dispatches=2 avg_us=3.000 median_us=3.000 min_us=2.000 max_us=4.000" in text
    assert "dispatches=1 avg_us=10.000" in text
