"""Host logic of bench.py (CPU only): the one-GPU refusal and the grid the
roofline's traffic lookup keys on."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_unit_grid_matches_the_launch_caps():
    # 21504 x 5376: 21 units per row, 3 rows per pass, 7168 passes, 4 waves
    # per workgroup -> 1792 workgroups, capped at 3 per CU for one matrix
    # and at 8 per CU for the pair
    assert bench.unit_grid(21504, 5376, 256, 3) == 768
    assert bench.unit_grid(21504, 5376, 256, 8) == 1792
    # 4096 x 4096: 4 rows per pass, 1024 passes -> 256 workgroups
    assert bench.unit_grid(4096, 4096, 256, 3) == 256
    assert bench.KERNEL_OF["qmv_q4_0"][1] == 3 and bench.KERNEL_OF["qmv_q4_0_geglu"][1] == 8


def test_traffic_is_withheld_for_an_unprofiled_grid():
    sym = bench.KERNEL_OF["qmv_q4_0_geglu"][0]
    assert bench.profiled_traffic(sym, 12345) is None


def test_trace_summary_reports_the_warm_mean(tmp_path):
    """The machine-readable trace mean is the mean of the calls that start
    50 ms or more after the kernel's first call (the state bench.py times in),
    and the plain mean for a kernel that ran for less than that."""
    import re
    ms = 1_000_000  # ns
    rows = []
    # kernel A: 10 cold calls of 30 us in the first 50 ms, then 10 warm ones of 20 us
    for i in range(10):
        rows.append(("void qmv::(anonymous namespace)::ka<1>(int)", i * 4 * ms, 30_000))
    for i in range(10):
        rows.append(("void qmv::(anonymous namespace)::ka<1>(int)", 60 * ms + i * ms, 20_000))
    # kernel B: three calls within 1 ms
    for i in range(3):
        rows.append(("void qmv::(anonymous namespace)::kb(float)", 70 * ms + i * 100_000, 5_000 + 1_000 * i))
    path = tmp_path / "run_kernel_trace.csv"
    with open(path, "w") as f:
        f.write("Kernel_Name,Start_Timestamp,End_Timestamp,Grid_Size_X,Workgroup_Size_X\n")
        for name, start, dur in rows:
            f.write(f'"{name}",{start},{start + dur},{256 * 768},256\n')
    text = bench.trace_summary(str(tmp_path), "cmd")
    marks = dict(((k, int(g)), float(v)) for k, g, v in
                 re.findall(r"<!-- trace (.+?) grid=(\d+) mean_us=([0-9.]+) -->", text))
    assert marks[("qmv::ka<1>", 768)] == 20.0
    assert abs(marks[("qmv::kb", 768)] - 6.0) < 1e-9
    assert "| `qmv::ka<1>` | 768 | 20 | 25.00 |" in text
