"""bench.py on the CPU: the one-GPU guard, the traffic-file lookup and the mixed MFMA peak (no device needed)."""
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


def test_mixed_mfma_peak_of_the_fp8_workloads():
    """The fp8 workloads' roofline peak weighs each contraction by its dtype: per key and
    head, 576 score columns at the fp8 peak (512 with the bf16 rope of R8) and the other
    columns (rope, 512 values) at the bf16 peak; bf16 workloads keep the bf16 peak."""
    import bench
    assert bench.mfma_peak("C1") == bench.BF16_PEAK_TFLOPS
    # time per flop column: 576 / 5000 + 512 / 2500 -> 1088 / 0.32 = 3400
    assert abs(bench.mfma_peak("D8") - 3400.0) < 1e-9
    assert bench.mfma_peak("C4") == bench.mfma_peak("D8") == bench.mfma_peak("S2")
    # R8: 512 fp8 columns, 64 + 512 bf16 columns -> 1088 / (0.1024 + 0.2304)
    assert abs(bench.mfma_peak("R8") - 1088 / (512 / 5000 + 576 / 2500)) < 1e-9
    assert bench.BF16_PEAK_TFLOPS < bench.mfma_peak("R8") < bench.mfma_peak("D8") < bench.FP8_PEAK_TFLOPS
