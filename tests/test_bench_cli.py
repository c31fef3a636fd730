"""CPU checks of bench.py's contract that need no GPU: more than one GPU is
refused with a message and a non-zero status before any device is touched,
and the committed HBM-traffic summary still matches the kernel sources (so
the benchmark line carries measured traffic rather than null)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "4"],
                         capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert res.returncode == 2
    assert "one GPU" in res.stdout


def test_traffic_summary_matches_kernel_sources():
    sys.path.insert(0, ROOT)
    import bench

    assert bench.measured_traffic("gemm_blockwise[t256x256bw16]") is not None, (
        "the GEMM sources changed since profiles/*_traffic.txt was taken: re-take FETCH_SIZE and "
        "WRITE_SIZE with rocprofv3 (commands in that file)")
