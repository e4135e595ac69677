"""Host-side checks of bench.py (no GPU): the one-GPU guard and the rule that
the counter-measured HBM traffic is reported only for the kernel sources it
was measured on."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402  (imports no GPU library at module level)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "exactly one GPU" in r.stderr


def test_traffic_only_for_the_measured_sources(monkeypatch):
    t = dict(bench.FORWARD_TRAFFIC)
    t.update(source_sha256=bench.kernel_sources_sha256(), fetch_kib=100.0, fetch_scale=2.0,
             write_kib=10.0, write_scale=1.0)
    monkeypatch.setattr(bench, "FORWARD_TRAFFIC", t)
    assert bench.forward_traffic(t["workload"], True) == (100 * 2 + 10) * 1024
    # another workload, the separate-prep kernel, or changed sources: no figure
    assert bench.forward_traffic("864x480_141f", True) is None
    assert bench.forward_traffic(t["workload"], False) is None
    monkeypatch.setitem(t, "source_sha256", "0" * 64)
    assert bench.forward_traffic(t["workload"], True) is None


def test_mixed_peak_is_the_harmonic_mean_of_the_halves():
    assert bench.mixed_peak(False, False) == pytest.approx(bench.PEAK_BF16_TFLOPS)
    hm = 2 / (1 / bench.PEAK_BF16_TFLOPS + 1 / bench.PEAK_FP8_TFLOPS)
    assert bench.mixed_peak(False, True) == pytest.approx(hm)
    assert bench.mixed_peak(True, True) == pytest.approx(bench.PEAK_INT8_TOPS)
