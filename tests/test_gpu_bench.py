"""bench.py end to end on the GPU: the one JSON line keeps its contract (the
metric and unit, whole-job value, steps, the roofline object with its live
timing, the traffic figure from the committed profile when the kernel code is
unchanged, the config naming the workload)."""
import json
import os
import subprocess
import sys

import pytest
import torch

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench(*args):
    print("[gpu case] bench.py", *args, flush=True)
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                       capture_output=True, text=True, timeout=240)
    assert p.returncode == 0, p.stderr[-2000:]
    lines = [l for l in p.stdout.splitlines() if l.strip()]
    assert len(lines) == 1, p.stdout
    return json.loads(lines[0])


def test_bench_line_contract():
    d = _bench("--steps", "3", "--warmup", "1", "--no-cpu-baseline", "--timed-only")
    assert d["metric"].startswith("ms/attn layer + effective TFLOPS")
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1
    assert d["higher_is_better"] is True and d["dtype"] == "bf16"
    assert d["value"] > 0 and d["ms_per_step"] > 0
    assert d["vs_baseline"] is None
    assert d["config"]["workload"].startswith("wan22-14b-480p")
    r = d["roofline"]
    assert r["bound"] == "mfma" and r["peak"] == 2500.0 and r["unit"] == "TFLOP/s"
    assert abs(r["frac"] - r["achieved"] / r["peak"]) < 1e-3
    assert r["traffic"] is None or r["traffic"] > 1e9
    # the whole layer is slower than its attention kernel alone
    assert d["ms_per_step"] >= d["ms_attend_kernel"]


def test_bench_mfma_probe():
    d = _bench("--mfma-peak", "--probe-launches", "2")
    runs = d["mfma_probe_bf16"]
    assert [p["waves_per_simd"] for p in runs] == [1, 2, 3]
    for p in runs:
        assert 100.0 < p["tflops"] < 2600.0
    loops = d["attn_loop_probe"]
    assert [p["queries_per_wave"] for p in loops] == [32, 64]
    for p in loops:
        assert 100.0 < p["tflops"] < 2600.0
