"""bench.py's output contract: one JSON line with the metric, the roofline of
the dominant kernel and the oracle's host baseline; one GPU only."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_cpu_baseline_reports_the_oracle_on_a_bounded_sample():
    import bench
    import synth
    w = synth.WORKLOADS["tiny"]
    cb = bench.cpu_baseline(w, 0.2)
    assert cb["kind"] == "oracle"
    assert cb["unit"] == "TFLOP/s"
    assert cb["value"] > 0
    assert cb["cores"] >= 1
    assert cb["calls"] >= 1
    assert "tiny" in cb["sample"]
    # FLOPs of one call: 4 * queries * |S| * d * H over the measured time
    from oracle import attention as O1
    kv_len = O1.kv_length(w.window + 1, w.cond_tokens, w.chunk_tokens, w.window)
    flops = 4.0 * w.chunk_tokens * kv_len * w.head_dim * w.heads * cb["calls"]
    assert cb["value"] == pytest.approx(flops / cb["seconds"] / 1e12, rel=1e-9)


def test_cpu_baseline_legs():
    # one core, the fp8 configuration's oracle and the full-depth
    # extrapolation, each labelled; the fp8 leg needs the 720p shape, so on
    # the tiny workload it is absent
    import bench
    import synth
    w = synth.WORKLOADS["tiny"]
    cb = bench.cpu_baseline(w, 0.2, legs=True)
    legs = cb["legs"]
    assert legs["single_core"]["cores"] == 1 and legs["single_core"]["value"] > 0
    assert "fp8" not in legs
    d = legs["depth_extrapolated"]
    assert d["extrapolated"] is True and d["unit"] == "chunks/s"
    assert d["chunks_per_s"] == pytest.approx(cb["chunks_per_s"] / 96)


def test_shader_clock_parsing():
    import bench
    assert bench.sclk_mhz({"sclk clock speed:": "(2100Mhz)", "sclk clock level:": "1"}) == 2100
    assert bench.sclk_mhz({"Temperature (Sensor edge) (C)": "41.0"}) is None
    assert bench.sclk_mhz(None) is None


@pytest.mark.gpu
def test_bench_line_on_the_tiny_workload():
    print("bench.py --config tiny --steps 3", flush=True)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--config", "tiny",
                        "--steps", "3", "--warmup", "1", "--warmup-ms", "20",
                        "--no-cpu-baseline"],
                       capture_output=True, text=True, timeout=240)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.startswith("{")]
    assert len(lines) == 1
    j = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "roofline"):
        assert key in j, key
    assert j["n_gpus"] == 1 and j["steps"] == 3 and j["warmup"] == 1
    assert j["value"] > 0 and j["ms_per_step"] > 0
    assert j["higher_is_better"] is True
    assert j["dtype"] == "bf16"
    assert "workload" in j["config"] and "model" not in j["config"]
    rf = j["roofline"]
    assert rf["bound"] == "mfma" and rf["unit"] == "TFLOP/s"
    assert rf["peak"] == pytest.approx(2516.6)
    # frac is printed with 4 decimals
    assert abs(rf["frac"] - rf["achieved"] / rf["peak"]) <= 5e-5 + 1e-9
    assert "cpu_baseline" not in j
    # the shader clock read under load (None if rocm-smi gives none), and the
    # roofline fraction at that clock
    assert "sclk_mhz_under_load" in j
    mhz = j["sclk_mhz_under_load"]
    if mhz:
        assert 500 <= mhz <= 3000
        assert rf["frac_at_measured_clock"] == pytest.approx(
            rf["achieved"] / (rf["peak"] * mhz / 2400), abs=1e-4)
