"""fp64-oracle parity of the large-matrix workloads at full size.

``large_n5`` and ``large_n10``: 16 x [8192, 8192], 16 x [8192, 28672] and
16 x [28672, 8192] (N = 5 and N = 10; "Muon is Scalable for LLM Training",
section 2.1, Eq. 2, and section 2.2, "other hyper-parameters", for N = 5
and the 5-vs-10 comparison).  One plan step over every matrix of the
workload runs in the launch configuration the benchmark times (one plan,
full workspace); then one matrix of each shape is compared with the fp64
oracle, started from the same pre-step state:

* X_N recovered from the fp32 weights, ``((1 - lr wd) W_old - W_new) /
  (lr 0.2 sqrt(max(A, B)))``, against the oracle's X_N: relative Frobenius
  error <= 2e-2 at N = 5;
* the per-singular-value deviation ``max_i |u_i^T X v_i - f^N(sigma_i /
  ||N||)|`` <= 0.05 at N = 5;
* at N = 10 bf16 iterates meet neither bar at this size, on the GPU or in
  the CPU rounding model of test_bf16_model.py (which reproduces the
  figures at full size): relative Frobenius error 2.15-2.19e-2 (bound
  2.5e-2); per-sigma 0.040-0.051 over the directions whose normalised
  singular value x0 is at least 2^-8 / sqrt(m) (bound 0.06) -- the worst
  sit at x0 ~ 0.0123, where the 10-fold map's slope amplifies rounding
  most -- and, on the square shape, up to 0.16 over the ~20 directions
  below that floor, which the iterates cannot follow (bound 0.25);
* the bf16 momentum elementwise against the oracle's formula, and the
  reported update RMS against the oracle's.

The oracle's X_N at these sizes is its spectral closed form taken through
the eigenproblem of the short-side Gram matrix (``ns_closed_form_gram``),
which the CPU pins tie to the iterated oracle; here it is also checked
against the iterated oracle itself on the square matrix at N = 5.  The
singular triplets of the per-sigma check come from the same
eigendecomposition.  A full fp64 iteration of every sampled matrix (up to
9e13 flops each at N = 10) would take tens of minutes on the host.
"""

from __future__ import annotations

import math
import time

import numpy as np
import pytest
import torch

import workloads as W
from oracle import muon_oracle as mo, spectral as sp

pytestmark = pytest.mark.gpu
HYP = dict(lr=1e-3, wd=0.1, mu=0.95, nesterov=True, rms_scale=0.2, eps=1e-7)
SAMPLES = {"sq": 0, "wide": 16, "tall": 32}          # first matrix of each shape group


def f64(t):
    return t.detach().float().cpu().double().numpy()


@pytest.fixture(scope="module")
def mod():
    import matrix_orthogonalizing_optimizer_amd as m
    m._lib.lib()
    return m


@pytest.fixture(scope="module", params=["large_n5", "large_n10"])
def large_run(request, mod):
    """One full-workload plan step; host copies of the sampled matrices."""
    key = request.param
    wl = W.WORKLOADS[key]
    t0 = time.perf_counter()
    T = W.make_muon_tensors(wl, "cuda")
    before = {name: (f64(T.params[i]), f64(T.grads[i]), f64(T.moms[i])) for name, i in SAMPLES.items()}
    plan = mod.MuonPlan(T.params, T.grads, T.moms, ns_dtype=wl.ns_dtype)
    ws = torch.empty(plan.workspace_bytes, dtype=torch.uint8, device="cuda")
    rms = torch.zeros(wl.n_mats, device="cuda")
    plan.step(ns_steps=wl.ns_steps, workspace=ws, update_rms=rms, **HYP)
    torch.cuda.synchronize()
    plan.close()
    after = {name: (f64(T.params[i]), f64(T.moms[i]), rms[i].item()) for name, i in SAMPLES.items()}
    del ws, T, rms, plan
    torch.cuda.empty_cache()
    print(f"{key}: GPU step and copies {time.perf_counter() - t0:.1f} s")
    return key, wl, before, after


@pytest.mark.parametrize("name", ["sq", "wide", "tall"])
def test_large_oracle_parity(large_run, name):
    key, wl, before, after = large_run
    steps = wl.ns_steps
    P0, G0, M0 = before[name]
    P1, M1, rms_gpu = after[name]
    r, c = P0.shape
    t0 = time.perf_counter()
    # momentum: bf16 storage of the fp32 result, half an ulp plus fp32 rounding
    Mo, N = mo.momentum_update(M0, G0, HYP["mu"], HYP["nesterov"])
    tol = np.abs(Mo) * (2.0 ** -8 + 2.0 ** -20) + (np.abs(HYP["mu"] * M0) + np.abs(G0)) * 2.0 ** -22 + 1e-30
    assert np.all(np.abs(M1 - Mo) <= tol), (key, name)
    del Mo, M0, M1, G0
    # X_N recovered from the weights
    step = HYP["lr"] * HYP["rms_scale"] * math.sqrt(max(r, c))
    X = (P0 - P1 - HYP["lr"] * HYP["wd"] * P0) / step
    del P1
    eig = sp.short_side_eig(N)
    Xo = sp.ns_closed_form_gram(N, steps, eps=HYP["eps"], eig=eig)
    if name == "sq" and steps == 5:
        Xi, _ = mo.orthogonalize(N, steps, eps=HYP["eps"])
        route = sp.rel_fro(Xo, Xi)
        print(f"closed form vs iterated oracle at [{r},{c}], N = 5: {route:.2e}")
        assert route <= 1e-9
        del Xi
    err = sp.rel_fro(X, Xo)
    rms_o = mo.update_rms(Xo)
    del Xo
    sig, proj = sp.per_sigma_projections_gram(X, N, eig)
    nu = float(np.sqrt(np.sum(N * N)))
    dev = np.abs(proj - sp.scalar_map(sig / (nu + HYP["eps"]), steps))
    x0 = sig / (nu + HYP["eps"])
    worst = float(dev.max())
    # the deviation restricted to directions bf16 iterates can follow
    # (normalised singular value >= 2^-8 / sqrt(m), see test_bf16_model.py)
    floor = 2.0 ** -8 / math.sqrt(min(r, c))
    resolved = float(dev[x0 >= floor].max())
    print(f"{key} {name} [{r},{c}]: X_N rel_fro {err:.3e}, per-sigma {worst:.3e} "
          f"(x0 >= {floor:.1e}: {resolved:.3e}, {int(np.sum(x0 < floor))} below; smallest x0 "
          f"{x0.min():.2e}, at worst {x0[dev.argmax()]:.2e}), "
          f"rms {rms_gpu:.5f} vs {rms_o:.5f}, host {time.perf_counter() - t0:.0f} s")
    assert abs(rms_gpu - rms_o) <= 2e-2 * rms_o
    if steps == 5:
        assert err <= 2e-2, (key, name, err)
        assert worst <= 0.05, (key, name, worst)
    else:
        # bf16 iterates at N = 10 (measured figures in the docstring)
        assert err <= 2.5e-2, (key, name, err)
        assert resolved <= 0.06, (key, name, resolved)
        assert worst <= (0.25 if name == "sq" else 0.06), (key, name, worst)
