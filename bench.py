"""Benchmark of the Muon optimizer step on one MI355X.

Default workload: the large-matrix step, the largest configuration that
fits one GPU -- 16 x [8192,8192], 16 x [8192,28672] and 16 x [28672,8192]
Muon matrices (fp32 weights, bf16 gradients, bf16 momentum, bf16
Newton-Schulz, N = 5).  ``--workload`` selects the others (the 800M-style
dense decoder with its AdamW side tensors, the 1.5B GQA model, the MoE
share, the per-head split, N = 10, the fp32 matrix).  Inputs are synthetic
(seeded) and resident in HBM before timing starts.

One JSON line is printed.  `value` is optimizer steps/s over the timed
steps (wall clock, synchronised on both sides).  The `roofline` object is
for the dominant kernel (the Newton-Schulz update GEMM X <- aX + PX): its
algorithmic flops per launch divided by its mean launch time, measured with
HIP events on the launch stream over the same timed steps.
`cpu_baseline` times the fp64 CPU oracle on a bounded sample of the same
workload -- one matrix of every shape group (the whole N-iteration step, or,
where that would take more than a few seconds, the step at N = 0 and N = 1,
extrapolated linearly to N) and one tensor per AdamW group -- and scales it
to the whole step by the group counts.  The roofline peaks are the
datasheet's; the line also carries the peaks measured on the GPU by the
probes of ``include/mo_probe.h`` (matrix cores alone, HBM streams alone).
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

BF16_PEAK_TFLOPS = 2516.6      # 256 CU x 4096 flop/clk x 2.4 GHz, dense
FP32_PEAK_TFLOPS = 157.3       # fp32 matrix
HBM_PEAK_GBS = 8000.0

HYPER = dict(lr=1e-3, wd=0.1, mu=0.95, nesterov=True, rms_scale=0.2, eps=1e-7)


def measured_traffic(name: str, match):
    """Calibrated HBM bytes per dispatch of the kernels whose names `match`
    accepts, from the committed rocprofv3 counter summary
    (profiles/hbm_traffic_<name>.json), or None when there is none or the
    kernel sources listed there changed since it was taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"hbm_traffic_{name}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    h = hashlib.sha256()
    for f in rec["sources"]:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    if h.hexdigest() != rec["source_sha256"]:
        return None
    n = b = 0.0
    for kname, k in rec["kernels"].items():
        if match(kname):
            n += k["dispatches"]
            b += k["dispatches"] * k["hbm_bytes_per_dispatch"]
    return b / n if n else None


def _is_small_kernel(name: str) -> bool:
    return name.startswith("mo::ns_small_kernel")


def _is_update_gemm(name: str) -> bool:
    # mo::ns_gemm_kernel<T, TILE, EPI, WAVES>, EPI 2 = the update product
    targs = name[name.find("<") + 1:name.rfind(">")].split(",")
    return name.startswith("mo::ns_gemm_kernel") and len(targs) > 2 and int(targs[2]) == 2


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="large_n5",
                    help="large_n5 (default), large_n10, dense800m, llama1p5b_gqa, moe_share, "
                         "fp32_128x512, kv_heads")
    ap.add_argument("--scaling", default="shape", choices=["shape", "hidden", "update_norm"],
                    help="update scaling: 0.2 sqrt(max(A,B)) (default), 0.2 sqrt(H) with H the "
                         "workload model's hidden size, or 0.2 / RMS(X_N)")
    ap.add_argument("--no-probe", action="store_true",
                    help="do not measure the matrix-core and HBM peaks")
    ap.add_argument("--svd-entropy", action="store_true",
                    help="time the SVD-entropy diagnostic (section 3.4) over the workload's "
                         "Muon weight matrices instead of the optimizer step")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-profile", action="store_true",
                    help="do not bracket launches with HIP events")
    return ap.parse_args()


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wl, muon_T, adam_T, direct_flops: float = 3e12):
    """Time the fp64 oracle on one matrix per shape group (and one tensor per
    AdamW group), scale by the group counts; returns the baseline dict.

    A group whose N-iteration oracle step exceeds ``direct_flops`` (dense
    count) is timed at N = 0 and N = 1 and extrapolated linearly to N: the
    iterations are identical, so the step costs t(0) + N (t(1) - t(0))."""
    from threadpoolctl import threadpool_info

    from oracle import muon_oracle as mo

    import workloads as W

    def f64(t):
        return t.detach().float().cpu().double().numpy()

    def timed(P, G, M, steps):
        t0 = time.perf_counter()
        mo.muon_step(P, G, M, ns_steps=steps, abc=mo.NS_COEFFS, **HYPER)
        return time.perf_counter() - t0

    t_total = 0.0
    sample = []
    idx = 0
    for grp in wl.mats:
        P, G, M = (f64(x[idx]) for x in (muon_T.params, muon_T.grads, muon_T.moms))
        _, dense = W.ns_flops(grp.rows, grp.cols, wl.ns_steps)
        if dense <= direct_flops:
            dt = timed(P, G, M, wl.ns_steps)
            sample.append(f"1 of {grp.count} [{grp.rows},{grp.cols}] ({dt:.2f} s)")
        else:
            t0 = timed(P, G, M, 0)
            t1 = timed(P, G, M, 1)
            dt = t0 + wl.ns_steps * max(t1 - t0, 0.0)
            sample.append(f"1 of {grp.count} [{grp.rows},{grp.cols}] at N=0 ({t0:.2f} s) and N=1 "
                          f"({t1:.2f} s), extrapolated to N={wl.ns_steps} ({dt:.1f} s)")
        t_total += dt * grp.count
        idx += grp.count
    if adam_T is not None:
        k = 0
        for vg in wl.vecs:
            p, g, m, v = (f64(x[k]) for x in (adam_T.params, adam_T.grads, adam_T.m, adam_T.v))
            t0 = time.perf_counter()
            mo.adamw_step(p, g, m, v, lr=HYPER["lr"], wd=HYPER["wd"], t=1)
            dt = time.perf_counter() - t0
            t_total += dt * vg.count
            sample.append(f"1 of {vg.count} AdamW {list(vg.shape)} ({dt:.3f} s)")
            k += vg.count
    threads = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
    return {"value": 1.0 / t_total, "unit": "steps/s", "cores": threads,
            "kind": "oracle", "cpu": cpu_model(),
            "sample": ("fp64 numpy oracle, full step scaled by the group counts from " + "; ".join(sample)
                       + f"; host has {len(os.sched_getaffinity(0))} usable cores")}


def measured_peaks():
    """The matrix-core and HBM rates the GPU sustains on their own
    (libmoprobe.so, include/mo_probe.h), or None when the probe library is
    missing or fails."""
    import ctypes
    path = os.path.join(ROOT, "matrix_orthogonalizing_optimizer_amd", "libmoprobe.so")
    if not os.path.exists(path):
        return None
    L = ctypes.CDLL(path)
    L.mo_probe_mfma_bf16.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.POINTER(ctypes.c_double)]
    L.mo_probe_mfma_bf16_random.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.POINTER(ctypes.c_double)]
    L.mo_probe_hbm.argtypes = [ctypes.c_size_t, ctypes.c_int, ctypes.POINTER(ctypes.c_double),
                               ctypes.POINTER(ctypes.c_double)]
    tf, tr, rd, cp = ctypes.c_double(), ctypes.c_double(), ctypes.c_double(), ctypes.c_double()
    if L.mo_probe_mfma_bf16(20000, 3, ctypes.byref(tf)) != 0:
        return None
    if L.mo_probe_mfma_bf16_random(20000, 3, ctypes.byref(tr)) != 0:
        return None
    if L.mo_probe_hbm(4 << 30, 3, ctypes.byref(rd), ctypes.byref(cp)) != 0:
        return None
    return {"bf16_mfma_tflops": tf.value, "bf16_mfma_random_tflops": tr.value,
            "hbm_read_gbs": rd.value, "hbm_copy_gbs": cp.value,
            "method": "register-only v_mfma_f32_32x32x16_bf16 loop, 2 waves per SIMD on every CU, on "
                      "near-constant operands and on random bf16 operands cycled per instruction; "
                      "4 GiB read-only and copy streams (copy counts read + write)"}


FP64_PEAK_TFLOPS = 78.6       # fp64 vector and matrix


def svd_main(args, torch, mo_amd, W, wl, dev):
    """SVD entropy and singular values of every Muon weight matrix of the
    workload (fp32 weights); a run is one mo_svd_entropy call over all of
    them.  The roofline is that of the reduction pass (rank-2 update and
    matrix-vector products of one Householder step), HBM-bound: its
    algorithmic bytes are the block-lower trailing elements it reads, 8
    bytes each."""
    T = W.make_muon_tensors(wl, dev)
    mats = list(T.params)
    full, _ = mo_amd.svd_entropy_workspace_size(tuple(x.shape) for x in mats)
    ws = torch.empty(full, dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    def run():
        return mo_amd.svd_entropy(mats, sigma=True, workspace=ws)

    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    classes = ["svd_gram", "svd_reduce", "svd_panel", "svd_column", "svd_eig"]
    mo_amd.profile_reset()
    if not args.no_profile:
        mo_amd.profile_enable(classes)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        h, _sig = run()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    mo_amd.profile_enable([])
    prof = {c: mo_amd.profile_read(c) for c in classes}
    ms_per_run = elapsed * 1e3 / args.steps
    kernels = {}
    for c in classes:
        n, ms, work = prof[c]
        if n:
            unit = {"svd_gram": "TFLOP/s", "svd_eig": "Gpivot/s"}.get(c, "GB/s")
            scale = {"TFLOP/s": 1e12, "Gpivot/s": 1e9, "GB/s": 1e9}[unit]
            rate = work / (ms * 1e-3) / scale if ms > 0 else None
            pk = {"TFLOP/s": FP64_PEAK_TFLOPS, "GB/s": HBM_PEAK_GBS}.get(unit)
            kernels[c] = {"launches": n, "ms_per_run": ms / args.steps, "mean_ms": ms / n,
                          "rate": rate, "unit": unit,
                          "frac": rate / pk if (rate is not None and pk) else None}
    red = prof["svd_reduce"]
    roofline = None
    if red[0]:
        ach = red[2] / (red[1] * 1e-3) / 1e9
        roofline = {"bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": ach / HBM_PEAK_GBS,
                    "traffic": measured_traffic(f"svd_entropy_{wl.key}",
                                                lambda n: n.endswith("svd_trd_pass_kernel")),
                    "kernel": "svd_trd_pass (matrix-vector products of one Householder step)",
                    "bytes_per_launch": red[2] / red[0], "mean_launch_ms": red[1] / red[0]}
    line = {
        "metric": "SVD-entropy diagnostic matrices/s (section 3.4 entropy + appendix F spectrum)",
        "value": len(mats) * 1e3 / ms_per_run, "unit": "matrices/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_run,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f64",
        "data": "synthetic (seeded random-init fp32 weights of the workload)",
        "config": {"workload": wl.key, "matrices": len(mats),
                   "shapes": sorted({f"{g.rows}x{g.cols}" for g in wl.mats})},
        "entropy_mean": float(h.mean()),
        "kernels": kernels,
        "roofline": roofline,
    }
    if not args.no_cpu_baseline:
        from threadpoolctl import threadpool_info

        from oracle import svd_entropy as se
        t_total, sample, idx = 0.0, [], 0
        for grp in wl.mats:
            w = mats[idx].detach().cpu().double().numpy()
            t1 = time.perf_counter()
            se.svd_entropy(w)
            dt = time.perf_counter() - t1
            t_total += dt * grp.count
            sample.append(f"1 of {grp.count} [{grp.rows},{grp.cols}] ({dt:.2f} s)")
            idx += grp.count
        threads = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
        line["cpu_baseline"] = {
            "value": len(mats) / t_total, "unit": "matrices/s", "cores": threads, "kind": "oracle",
            "sample": ("fp64 numpy SVD oracle, extrapolated from " + "; ".join(sample)
                       + f"; host has {len(os.sched_getaffinity(0))} usable cores")}
    print(json.dumps(line), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(the step runs whole matrices on one GPU, with no sharding or collectives)", file=sys.stderr)
        sys.exit(2)
    import torch

    import matrix_orthogonalizing_optimizer_amd as mo_amd
    import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wl = W.WORKLOADS[args.workload]
    mo_amd._lib.lib()
    if args.svd_entropy:
        svd_main(args, torch, mo_amd, W, wl, dev)
        return

    T = W.make_muon_tensors(wl, dev)
    A = W.make_adamw_tensors(wl, dev) if wl.vecs else None
    plan = mo_amd.MuonPlan(T.params, T.grads, T.moms, ns_dtype=wl.ns_dtype)
    ws = torch.empty(plan.workspace_bytes, dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    step_no = [0]

    hidden = float(wl.hidden)

    def opt_step():
        step_no[0] += 1
        plan.step(ns_steps=wl.ns_steps, workspace=ws, scaling=args.scaling, hidden=hidden, **HYPER)
        if A is not None:
            mo_amd.adamw_step(A.params, A.grads, A.m, A.v, lr=HYPER["lr"], wd=HYPER["wd"],
                              step=step_no[0])

    for _ in range(args.warmup):
        opt_step()
    torch.cuda.synchronize()

    classes = ["momentum", "norm", "gram", "poly", "update", "apply", "rms", "adamw"]
    mo_amd.profile_reset()
    if not args.no_profile:
        mo_amd.profile_enable(classes)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        opt_step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    mo_amd.profile_enable([])
    prof = {c: mo_amd.profile_read(c) for c in classes}

    ms_per_step = elapsed * 1e3 / args.steps
    steps_per_s = 1e3 / ms_per_step
    alg_flops, dense_flops = W.workload_ns_flops(wl)
    ns_ms = sum(prof[c][1] for c in ("gram", "poly", "update", "apply")) / args.steps
    peak = BF16_PEAK_TFLOPS if wl.ns_dtype == torch.bfloat16 else FP32_PEAK_TFLOPS
    kernels = {}
    for c in classes:
        n, ms, work = prof[c]
        if n:
            unit = "TFLOP/s" if c in ("gram", "poly", "update", "apply") else "GB/s"
            rate = work / (ms * 1e-3) / (1e12 if unit == "TFLOP/s" else 1e9)
            kernels[c] = {"launches": n, "mean_ms": ms / n, "rate": rate, "unit": unit,
                          "frac": rate / (peak if unit == "TFLOP/s" else HBM_PEAK_GBS)}
    upd = prof["update"]
    peaks = None if args.no_probe else measured_peaks()
    roofline = None
    # groups of small matrices (m <= 128) run one fused kernel per step,
    # recorded as the update class with no Gram, polynomial or apply
    # launches; it moves X_0 twice (bf16) and W in and out (fp32) and is
    # bound by HBM, not by the matrix cores
    fused_small = upd[0] > 0 and prof["gram"][0] == 0 and prof["apply"][0] == 0
    if fused_small and wl.ns_dtype == torch.bfloat16:
        fbytes = wl.n_elems * (2 * 2 + 8) * args.steps          # over the timed steps
        ach = fbytes / (upd[1] * 1e-3) / 1e9
        kernels["update"]["hbm_gb_per_s"] = ach
        roofline = {"bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": ach / HBM_PEAK_GBS, "traffic": measured_traffic(wl.key, _is_small_kernel),
                    "kernel": "ns_small fused Newton-Schulz + apply (Gram-space iteration)",
                    "bytes_per_launch": fbytes / upd[0], "mean_launch_ms": upd[1] / upd[0],
                    "alg_tflops": upd[2] / (upd[1] * 1e-3) / 1e12}
        if peaks:
            roofline["measured_peak"] = peaks["hbm_copy_gbs"]
            roofline["frac_of_measured_peak"] = ach / peaks["hbm_copy_gbs"]
    elif upd[0]:
        ach = upd[2] / (upd[1] * 1e-3) / 1e12
        roofline = {"bound": "mfma", "achieved": ach, "peak": peak, "unit": "TFLOP/s",
                    "frac": ach / peak, "traffic": measured_traffic(wl.key, _is_update_gemm),
                    "kernel": "ns_gemm update X <- aX + PX",
                    "flops_per_launch": upd[2] / upd[0], "mean_launch_ms": upd[1] / upd[0]}
        if peaks and wl.ns_dtype == torch.bfloat16:
            roofline["measured_peak"] = peaks["bf16_mfma_tflops"]
            roofline["frac_of_measured_peak"] = ach / peaks["bf16_mfma_tflops"]
            roofline["measured_peak_random_operands"] = peaks["bf16_mfma_random_tflops"]
            roofline["frac_of_measured_peak_random_operands"] = ach / peaks["bf16_mfma_random_tflops"]
    if peaks:
        for k in kernels.values():
            if k["unit"] == "GB/s":
                k["frac_of_measured_copy"] = k["rate"] / peaks["hbm_copy_gbs"]
    ew_bytes = wl.n_elems * W.muon_elementwise_bytes_per_elem(wl) + \
        (wl.n_vec_elems * W.ADAMW_BYTES_PER_ELEM if wl.vecs else 0)
    ideal_ms = (alg_flops / (peak * 1e12) + ew_bytes / (HBM_PEAK_GBS * 1e9)) * 1e3
    line = {
        "metric": "Muon optimizer steps/s + Newton-Schulz TFLOP/s (% bf16 MFMA peak) per config",
        "value": steps_per_s, "unit": "steps/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if wl.ns_dtype == torch.bfloat16 else "f32",
        "data": "synthetic (seeded; random-init weights, Gaussian gradients)",
        "config": {"workload": wl.key, "muon_matrices": wl.n_mats,
                   "muon_elements": wl.n_elems, "adamw_elements": wl.n_vec_elems,
                   "ns_steps": wl.ns_steps, "scaling": args.scaling,
                   "grad_dtype": str(wl.grad_dtype).split(".")[-1],
                   "mom_dtype": str(wl.mom_dtype).split(".")[-1],
                   "seeds": {"weights": W.seed_of(wl.cid, 0), "grads": W.seed_of(wl.cid, 1),
                             "rule": "workload id x 1e6 + tensor kind x 1e4 + step "
                                     "(kinds: 0 W, 1 G, 2 M, 3 scales, 4 AdamW W, 5 AdamW g)"}},
        "matrices_per_s": wl.n_mats * steps_per_s,
        "ns_alg_tflop_per_step": alg_flops / 1e12,
        "ns_tflops": (alg_flops / (ns_ms * 1e-3) / 1e12) if ns_ms > 0 else None,
        "ns_frac_peak": (alg_flops / (ns_ms * 1e-3) / 1e12 / peak) if ns_ms > 0 else None,
        "ns_ms_per_step": ns_ms,
        "step_tflops_wallclock": alg_flops / (ms_per_step * 1e-3) / 1e12,
        "elementwise_alg_gb_per_step": ew_bytes / 1e9,
        # the step at the datasheet roofline: products at the MFMA peak,
        # momentum/apply/AdamW bytes at 8 TB/s
        "ideal_step_ms": ideal_ms,
        "frac_of_ideal_step_rate": ideal_ms / ms_per_step,
        "kernels": kernels,
        "roofline": roofline,
        "measured_peaks": peaks,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(wl, T, A)
    print(json.dumps(line), flush=True)
    plan.close()


if __name__ == "__main__":
    main()
