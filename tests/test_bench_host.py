"""bench.py on the CPU: the one-GPU guard and the traffic-file lookup (no device needed)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2, r.stderr
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""  # no JSON line for a configuration that was not run


def test_traffic_lookup_is_keyed_by_workload_and_sources():
    import bench
    assert bench.read_traffic("C2") is None  # counters are recorded for C1 only
    d1, d2 = bench.kernel_digest(), bench.kernel_digest()
    assert d1 == d2 and len(d1) == 16
