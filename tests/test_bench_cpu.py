"""Host-side checks of bench.py that need no GPU: it refuses more than one
GPU before touching a device, and it reports the LM-head kernel's counted
HBM traffic only while the committed counter summary was taken on the
current kernel source."""
import importlib.util
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench_module():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_counter_traffic_follows_the_kernel_source(monkeypatch):
    bench = _bench_module()
    path = os.path.join(ROOT, "profiles", "k1_lmhead_qwen3_4b_counters.json")
    with open(path) as f:
        c = json.load(f)
    # the summary's own figures hang together: counted bytes = scaled fetch + write
    cal = c["calibration"]
    assert abs(cal["fetch_scale"] - 0.50005) < 1e-3 and cal["write_scale"] == 1.0
    expect = c["fetch_kib_per_launch"] * 1024 / cal["fetch_scale"] + c["write_kib_per_launch"] * 1024
    assert abs(c["hbm_bytes_per_launch"] - expect) / expect < 1e-4
    assert c["hbm_bytes_per_launch"] >= c["algorithmic_bytes_per_launch"]
    # reported for the recorded source, withheld for any other
    monkeypatch.setattr(bench, "_src_sha", lambda p: c["kernel_src_sha"])
    assert bench.counters_traffic("qwen3_4b") == c["hbm_bytes_per_launch"]
    monkeypatch.setattr(bench, "_src_sha", lambda p: "0" * 16)
    assert bench.counters_traffic("qwen3_4b") is None
    assert bench.counters_traffic("no_such_workload") is None


def test_dominant_kernel_follows_the_path_each_workload_runs():
    import synth
    bench = _bench_module()
    k = {n: bench.dominant_kernel(c) for n, c in synth.CONFIGS.items()}
    assert k["qwen3_4b"]["kernel"] == "k1_lmhead_bf16" and k["qwen3_4b"]["bound"] == "hbm"
    assert k["wide"]["kernel"] == "k1_lmhead_bf16"
    # 128 hidden rows: the tiled product in 128 x 320 tiles, 128 flop per
    # weight byte, HBM-bound
    assert k["qwen3_8b_x8"]["kernel"] == "k_mm_lm<128, 320>" and k["qwen3_8b_x8"]["bound"] == "hbm"
    # 512 hidden rows: 128 x 256 tiles, past the ridge of the published
    # peaks, MFMA-bound
    assert k["stress_b0"]["kernel"] == "k_mm_lm<256, 256>"
    assert k["stress_b0"]["bound"] == "mfma" and k["stress_b0"]["unit"] == "TFLOP/s"
    c = synth.CONFIGS["stress_b0"]
    assert k["stress_b0"]["work"] == 2 * c.batch * c.D * c.d * c.V
