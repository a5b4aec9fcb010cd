"""Host-side checks of the benchmark and its synthetic workloads (no GPU).

* The workloads reproduce the configurations' sizes: matrix counts, Muon
  and AdamW element counts, and the algorithmic Newton-Schulz flops per step
  (3 m^2 n + m^3 per matrix and iteration, m = min side).
* ``bench.py --gpus N`` with N > 1 exits with a message (the step runs on one GPU).
* The calibrated-traffic lookup returns bytes only while the sha256 of the
  kernel sources it lists matches the tree, and None once they change.
"""

from __future__ import annotations

import hashlib
import json
import os
import subprocess
import sys

import pytest

import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("key,mats,elems,vec_elems,tflop", [
    ("fp32_128x512", 1, 65536, 0, 1.36315e-4),     # 5 (3 128^2 512 + 128^3) flops
    ("dense800m", 144, 679477248, 98379264, 18.26),
    ("llama1p5b_gqa", 168, 1082130432, 0, 37.27),
    ("moe_share", 1568, 4488953856, 0, 116.6),
    ("large_n5", 48, 8589934592, 0, 1187.0),
    ("large_n10", 48, 8589934592, 0, 2375.0),
])
def test_workload_sizes(key, mats, elems, vec_elems, tflop):
    wl = W.WORKLOADS[key]
    assert wl.n_mats == mats
    assert wl.n_elems == elems
    assert wl.n_vec_elems == vec_elems
    alg, dense = W.workload_ns_flops(wl)
    assert abs(alg / 1e12 - tflop) <= 2e-3 * tflop
    assert dense > alg


def test_ns_flops_formula():
    # one [4, 8] matrix, N = 5: 5 (3 * 4^2 * 8 + 4^3) = 2240
    wl = W.Workload(key="t", description="t", cid=99,
                    mats=(W.MatGroup("t", 8, 4, 1),), vecs=(), ns_steps=5,
                    grad_dtype=W.WORKLOADS["dense800m"].grad_dtype,
                    mom_dtype=W.WORKLOADS["dense800m"].mom_dtype,
                    ns_dtype=W.WORKLOADS["dense800m"].ns_dtype)
    assert W.workload_ns_flops(wl)[0] == 5 * (3 * 4 * 4 * 8 + 4 ** 3)


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr or "single" in r.stderr


def test_traffic_lookup_follows_the_source_hash(tmp_path, monkeypatch):
    import bench

    src = tmp_path / "k.hip"
    src.write_text("kernel v1\n")
    prof = tmp_path / "profiles"
    prof.mkdir()
    rec = {"sources": ["k.hip"],
           "source_sha256": hashlib.sha256(src.read_bytes()).hexdigest(),
           "kernels": {"mo::ns_gemm_kernel<unsigned short, 256, 2, 8>":
                       {"dispatches": 4, "hbm_bytes_per_dispatch": 1000.0},
                       "mo::ns_gemm_kernel<unsigned short, 256, 3, 8>":
                       {"dispatches": 1, "hbm_bytes_per_dispatch": 9.0}}}
    (prof / "hbm_traffic_w.json").write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.measured_traffic("w", bench._is_update_gemm) == 1000.0
    assert bench.measured_traffic("missing", bench._is_update_gemm) is None
    src.write_text("kernel v2\n")
    assert bench.measured_traffic("w", bench._is_update_gemm) is None


def test_committed_profiles_name_existing_sources():
    pdir = os.path.join(ROOT, "profiles")
    for f in os.listdir(pdir):
        if f.startswith("hbm_traffic_") and f.endswith(".json"):
            rec = json.load(open(os.path.join(pdir, f)))
            assert rec["sources"], f
            for s in rec["sources"]:
                assert os.path.exists(os.path.join(ROOT, s)), (f, s)
            assert rec["kernels"], f


def test_cpu_baseline_covers_every_group_and_extrapolates():
    """Every shape group is timed (none dropped on a budget); a group above
    the direct-timing threshold is timed at N = 0 and N = 1 and extrapolated,
    and says so; the CPU model is recorded."""
    import bench

    wl = W.Workload(key="t", description="t", cid=98,
                    mats=(W.MatGroup("a", 64, 96, 3), W.MatGroup("b", 160, 96, 2)),
                    vecs=(W.VecGroup("v", (40,), 2),), ns_steps=5,
                    grad_dtype=W.WORKLOADS["dense800m"].grad_dtype,
                    mom_dtype=W.WORKLOADS["dense800m"].mom_dtype,
                    ns_dtype=W.WORKLOADS["dense800m"].ns_dtype)
    T = W.make_muon_tensors(wl, "cpu")
    A = W.make_adamw_tensors(wl, "cpu")
    a_flops = W.ns_flops(64, 96, 5)[1]
    out = bench.cpu_baseline(wl, T, A, direct_flops=a_flops)     # group b above it
    assert out["kind"] == "oracle" and out["value"] > 0 and out["cores"] >= 1
    assert out["cpu"]
    s = out["sample"]
    assert "1 of 3 [64,96] (" in s
    assert "1 of 2 [160,96] at N=0" in s and "extrapolated to N=5" in s
    assert "1 of 2 AdamW [40]" in s


def test_eq5_hidden_size_is_the_model_width():
    """Section 3.1, Eq. 5 scales by 0.2 sqrt(H) with H the model's hidden
    size -- not the largest matrix side (6144 for the 800M MLP)."""
    assert W.WORKLOADS["dense800m"].hidden == 1536
    assert W.WORKLOADS["llama1p5b_gqa"].hidden == 2048
    assert W.WORKLOADS["moe_share"].hidden == 2048
    assert W.WORKLOADS["large_n5"].hidden == 8192
    src = open(os.path.join(ROOT, "bench.py")).read()
    assert "hidden = float(wl.hidden)" in src
