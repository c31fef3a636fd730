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
    """The committed counter summary is parsed, and it is used only while its
    source hash matches the kernels (else the bench line's traffic is null,
    which is reported here as a skip until the counters are re-taken)."""
    import glob

    import pytest

    sys.path.insert(0, ROOT)
    import bench

    files = glob.glob(os.path.join(ROOT, "profiles", "*_traffic.txt"))
    assert files, "no rocprofv3 FETCH_SIZE / WRITE_SIZE summary under profiles/"
    labels = {}
    for path in files:
        with open(path) as fh:
            kv = dict(line.rstrip("\n").split(": ", 1) for line in fh
                      if ": " in line and not line.startswith(" "))
        assert int(kv["traffic_bytes_per_launch"]) > 0 and int(kv["algorithmic_bytes_per_launch"]) > 0
        labels[kv["label"]] = kv["source_sha256"]
    current = bench.kernel_source_hash()
    for label, sha in labels.items():
        got = bench.measured_traffic(label)
        assert (got is not None) == (sha == current)
    if current not in labels.values():
        pytest.skip("the GEMM sources changed since profiles/*_traffic.txt was taken: the bench line "
                    "reports traffic null until FETCH_SIZE and WRITE_SIZE are re-taken (commands in that file)")
