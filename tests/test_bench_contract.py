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
