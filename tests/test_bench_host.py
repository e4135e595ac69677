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


def test_oracle_rows_recipe():
    from audio_video_diffusion_amd import workloads as W
    wl = W.WORKLOADS[W.HEADLINE]
    rows = bench.oracle_rows(wl, 2048)
    n = wl.n_tokens
    assert rows[0] == 0 and rows[-1] == n - 1 and len(set(rows.tolist())) == len(rows)
    assert set(range(64)) <= set(rows.tolist()) and set(range(n - 128, n)) <= set(rows.tolist())
    for b in (wl.video, wl.video + wl.audio):
        assert set(range(b - 8, b + 8)) <= set(rows.tolist())
    assert 2048 < len(rows) <= 2048 + 64 + 128 + 32
    assert len(bench.oracle_rows(W.WORKLOADS[0], 10 ** 6)) == W.WORKLOADS[0].n_tokens


def test_oracle_subset_whole_tiny_workload_and_extrapolation():
    from audio_video_diffusion_amd import workloads as W
    tiny = W.WORKLOADS[0]
    r = bench.oracle_subset(tiny, W.make_inputs(0), 16)
    assert r["full_s"] is not None and r["full_s_extrapolated"] is None
    assert r["rows"] == tiny.n_tokens and r["heads"] == tiny.heads
    wl = W.ragged_workload(5000, 3)
    r = bench.oracle_subset(wl, W.make_inputs(7, wl), 32, heads_n=1)
    assert r["full_s"] is None and r["heads"] == 1
    # the per-head prep of all keys counts once per head, the attention per row
    rows_s = r["seconds"] - r["prep_s"]
    expect = 3 * (r["prep_s"] + rows_s * 5000 / r["rows"])
    assert r["full_s_extrapolated"] == pytest.approx(expect, rel=0.01, abs=0.1)


def test_full_oracle_mode_on_the_tiny_workload(capsys):
    from audio_video_diffusion_amd import workloads as W
    bench.full_oracle(W, cfgs={0})
    import json
    out = json.loads(capsys.readouterr().out.strip().splitlines()[-1])
    assert out["workloads"][0]["whole"] and out["workloads"][0]["rows"] == W.WORKLOADS[0].n_tokens
    assert out["workers"] >= 1 and "cpu_count" in out["host"]
    # 4 heads x 2 row blocks: every head prepared at least once, at most once per unit
    assert 4 <= out["workloads"][0]["head_preps"] <= 8


def test_clock_sampler_reads_the_starred_level(tmp_path):
    f = tmp_path / "pp_dpm_sclk"
    f.write_text("0: 500Mhz\n1: 2400Mhz *\n")
    c = bench.ClockSampler(period_s=0.01)
    c.paths = [str(f)]
    with c:
        import time
        time.sleep(0.05)
    sm = c.summary()
    assert sm["median"] == 2400 and sm["samples"] >= 1
    c2 = bench.ClockSampler()
    c2.paths = [str(tmp_path / "missing")]
    with c2:
        pass
    assert c2.summary() is None


def test_code_hash_ignores_comments_only(tmp_path, monkeypatch):
    src = os.path.join(bench.ROOT, "audio_video_diffusion_amd", "csrc")
    dst = tmp_path / "audio_video_diffusion_amd" / "csrc"
    dst.mkdir(parents=True)
    texts = {n: open(os.path.join(src, n), encoding="utf-8").read() for n in ("forward.hip", "rope_norm.h")}
    base = bench.kernel_sources_sha256()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))

    def digest(fwd):
        (dst / "forward.hip").write_text(fwd, encoding="utf-8")
        (dst / "rope_norm.h").write_text(texts["rope_norm.h"], encoding="utf-8")
        return bench.kernel_sources_sha256()

    assert digest(texts["forward.hip"]) == base
    # comments and line breaks added: same code, same digest
    assert digest("// a note\n" + texts["forward.hip"].replace("\n", "\n\n", 3) + "\n/* end */\n") == base
    # a changed constant: another digest
    assert "kRescaleLog2 = 8.0f" in texts["forward.hip"]
    assert digest(texts["forward.hip"].replace("kRescaleLog2 = 8.0f", "kRescaleLog2 = 7.0f")) != base
