"""Host-side pieces of bench.py (no GPU): the multi-GPU refusal and the
algorithmic byte count of the headline workload."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_method_bytes_9b_t2048():
    """fwd + bwd bytes of the 9B layer at T=2048 (bf16 I/O, fp32 state and
    31 checkpoints): 660.1 MB, i.e. 82.5 us at 8 TB/s."""
    fb, bb = bench.method_bytes(1, 2048, 16, 64, 192, 128, 2)
    assert abs((fb + bb) / 1e6 - 660.1) < 0.1
    assert abs(fb / 1e6 - 300.4) < 0.1


def test_compulsory_bytes_9b_t2048():
    """Without the checkpoints the 9B layer at T=2048 moves 270.0 MB per step."""
    assert abs(bench.compulsory_bytes(1, 2048, 16, 64, 192, 128, 2) / 1e6 - 270.0) < 0.1


def test_stats_median_min_max():
    s = bench._stats([3.0, 1.0, 2.0, 10.0])
    assert s["median"] == 2.5 and s["min"] == 1.0 and s["max"] == 10.0 and s["mean"] == 4.0
    assert bench._stats([5.0, 1.0, 4.0])["median"] == 4.0
