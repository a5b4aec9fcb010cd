"""The benchmark's output contract on the GPU: one JSON line with the
required keys, a roofline object for the dominant kernel, and the oracle's
CPU baseline (default run); the SVD-entropy mode likewise."""

from __future__ import annotations

import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
KEYS = {"metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
        "scaling", "vs_baseline", "dtype", "data", "config", "roofline"}
ROOF = {"bound", "achieved", "peak", "unit", "frac", "traffic"}


def _run(args):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                       capture_output=True, text=True, timeout=600, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1, r.stdout
    return json.loads(lines[0])


def _check_common(d, steps, warmup):
    assert KEYS <= set(d), KEYS - set(d)
    assert d["n_gpus"] == 1 and d["steps"] == steps and d["warmup"] == warmup
    assert d["value"] > 0 and d["ms_per_step"] > 0 and d["higher_is_better"] is True
    assert "workload" in d["config"]
    roof = d["roofline"]
    assert ROOF <= set(roof), ROOF - set(roof)
    assert 0 < roof["frac"] < 1 and abs(roof["achieved"] / roof["peak"] - roof["frac"]) < 1e-9
    assert roof["traffic"] is None or roof["traffic"] > 0
    for name, k in d["kernels"].items():
        if k["unit"] in ("TFLOP/s", "GB/s"):
            assert 0 < k["frac"] < 1 and k["rate"] > 0, (name, k)


def test_bench_default_line():
    d = _run(["--steps", "2", "--warmup", "1"])
    _check_common(d, 2, 1)
    assert d["config"]["workload"] == "large_n5" and d["unit"] == "steps/s"
    assert d["roofline"]["bound"] == "mfma" and d["roofline"]["unit"] == "TFLOP/s"
    cpu = d["cpu_baseline"]
    assert cpu["kind"] == "oracle" and cpu["value"] > 0 and cpu["cores"] >= 1 and cpu["sample"]
    assert cpu["cpu"]
    for shape in ("[8192,8192]", "[8192,28672]", "[28672,8192]"):
        assert shape in cpu["sample"], shape
    pk = d["measured_peaks"]
    assert 500 < pk["bf16_mfma_tflops"] < 2600 and 1000 < pk["hbm_read_gbs"] < 9000
    assert 0 < d["roofline"]["frac_of_measured_peak"] < 1.2
    assert 500 < pk["bf16_mfma_random_tflops"] <= 1.05 * pk["bf16_mfma_tflops"]
    assert 0 < d["roofline"]["frac_of_measured_peak_random_operands"] < 1.2
    # the datasheet-roofline step: 1.187e15 flops at 2516.6 TFLOP/s plus 8.59e9
    # elements x 16 B at 8 TB/s
    assert abs(d["ideal_step_ms"] - (1.187e15 / 2516.6e12 + 8.59e9 * 16 / 8e12) * 1e3) < 2.0
    assert 0 < d["frac_of_ideal_step_rate"] < 1
    assert d["config"]["seeds"]["grads"] == 5 * 1_000_000 + 10_000


def test_bench_800m_line():
    d = _run(["--workload", "dense800m", "--steps", "2", "--warmup", "1", "--no-probe"])
    _check_common(d, 2, 1)
    assert d["config"]["workload"] == "dense800m" and "adamw" in d["kernels"]
    assert "[32000, 1536]" in d["cpu_baseline"]["sample"]


def test_bench_small_matrix_line():
    """The per-head workload runs the fused small-matrix kernel, which is
    bound by HBM: its roofline is GB/s over X_0 read twice and W read and
    written (12 bytes per element)."""
    d = _run(["--workload", "kv_heads", "--steps", "3", "--warmup", "1", "--no-probe", "--no-cpu-baseline"])
    _check_common(d, 3, 1)
    roof = d["roofline"]
    assert roof["bound"] == "hbm" and roof["unit"] == "GB/s" and "ns_small" in roof["kernel"]
    assert abs(roof["bytes_per_launch"] - 960 * 128 * 2048 * 12) < 1.0
    assert set(d["kernels"]) >= {"momentum", "update"} and "gram" not in d["kernels"]


def test_bench_svd_entropy_line():
    d = _run(["--svd-entropy", "--workload", "llama1p5b_gqa", "--steps", "1", "--warmup", "0",
              "--no-cpu-baseline"])
    _check_common(d, 1, 0)
    assert d["unit"] == "matrices/s" and d["dtype"] == "f64"
    assert d["roofline"]["bound"] == "hbm" and d["roofline"]["unit"] == "GB/s"
    assert 0.0 < d["entropy_mean"] <= 1.0
