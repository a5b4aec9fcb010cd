"""GPU parity of the HIP path against the fp64 oracle, through the C ABI.

Tolerances:
* fp32 Newton-Schulz path: relative Frobenius error of the update <= 1e-4;
* bf16 path: relative Frobenius error <= 2e-2 and per-singular-value
  deviation ``max_i |u_i^T X v_i - f^N(sigma_i)|`` <= 0.05 (singular
  vectors from the oracle's SVD of the Newton-Schulz input);
* momentum in bf16: within half a bf16 ulp of the oracle's fp64 value
  (round-to-nearest of the fp32 result); fp32 momentum to 1e-6 relative;
* AdamW: fp32 arithmetic against fp64, 1e-5 relative on the update.
bf16 inputs are upcast exactly for the oracle; the oracle always starts from
the same pre-step state as the GPU (step-local parity), except for the
all-fp32 workload whose three-step trajectory is compared directly.
"""

from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import workloads as W
from oracle import muon_oracle as mo, spectral as sp

pytestmark = pytest.mark.gpu

DEV = "cuda"
HYP = dict(lr=1e-3, wd=0.1, mu=0.95, nesterov=True, ns_steps=5, rms_scale=0.2, eps=1e-7)


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().double().numpy()


def _gen(seed):
    g = torch.Generator()
    g.manual_seed(seed)
    return g


def randn(shape, seed, std=1.0, dtype=torch.float32):
    return (torch.randn(*shape, generator=_gen(seed)) * std).to(dtype).to(DEV)


@pytest.fixture(scope="module")
def mod():
    import matrix_orthogonalizing_optimizer_amd as m
    m._lib.lib()
    return m


# ---------------------------------------------------------------- Newton-Schulz only

NS_F32_SHAPES = [(128, 512), (512, 128), (100, 300), (65, 64), (1, 40), (40, 1), (257, 130)]


@pytest.mark.parametrize("shape", NS_F32_SHAPES)
def test_ns_fp32(mod, shape):
    x = randn(shape, 1 + shape[0] * 3 + shape[1])
    X = mod.newton_schulz(x, ns_steps=5)
    torch.cuda.synchronize()
    ref, _ = mo.orthogonalize(f64(x), 5, eps=1e-7)
    assert sp.rel_fro(f64(X), ref) <= 1e-4


@pytest.mark.parametrize("steps", [0, 1, 2, 10])
def test_ns_fp32_steps(mod, steps):
    x = randn((96, 200), 7)
    X = mod.newton_schulz(x, ns_steps=steps)
    ref, _ = mo.orthogonalize(f64(x), steps, eps=1e-7)
    assert sp.rel_fro(f64(X), ref) <= 1e-4


NS_BF16_SHAPES = [(128, 512), (300, 700), (700, 300), (1408, 2048), (2048, 512),
                  (64, 2048), (512, 4096), (1536, 1536), (2048, 64), (257, 1031)]


@pytest.mark.parametrize("shape", NS_BF16_SHAPES)
def test_ns_bf16(mod, shape):
    x = randn(shape, 11 + shape[0] + 7 * shape[1], dtype=torch.bfloat16)
    X = mod.newton_schulz(x, ns_steps=5)
    xo = f64(x)
    ref, _ = mo.orthogonalize(xo, 5, eps=1e-7)
    err = sp.rel_fro(f64(X), ref)
    dev = sp.per_sigma_deviation(f64(X), xo, 5, eps=1e-7)
    print(f"{shape}: rel_fro {err:.3e} per_sigma {dev:.3e}")
    assert err <= 2e-2
    assert dev <= 0.05


def test_ns_bf16_thin_small_m(mod):
    """A 33 x 1000 input (no workload has it): storing S, P and X in bf16
    -- the precision the pages run Newton-Schulz in -- gives about 2.5e-2
    relative Frobenius error here (a CPU model of the same rounding points
    gives the same figure), so this shape is gated on the per-singular-value
    criterion, with a looser Frobenius bound."""
    x = randn((33, 1000), 11 + 33 + 7000, dtype=torch.bfloat16)
    X = mod.newton_schulz(x, ns_steps=5)
    xo = f64(x)
    ref, _ = mo.orthogonalize(xo, 5, eps=1e-7)
    assert sp.rel_fro(f64(X), ref) <= 3e-2
    assert sp.per_sigma_deviation(f64(X), xo, 5, eps=1e-7) <= 0.05


def test_ns_batched_bf16(mod):
    x = randn((6, 256, 384), 5, dtype=torch.bfloat16)
    X = mod.newton_schulz(x, ns_steps=5)
    for b in range(6):
        ref, _ = mo.orthogonalize(f64(x[b]), 5, eps=1e-7)
        assert sp.rel_fro(f64(X[b]), ref) <= 2e-2


def test_ns_zero_input(mod):
    x = torch.zeros(64, 192, device=DEV)
    X = mod.newton_schulz(x, ns_steps=5)
    assert torch.count_nonzero(X).item() == 0


# ---------------------------------------------------------------- full step, fp32

def test_fp32_workload_three_steps(mod):
    """The all-fp32 workload: [128,512], W~N(0,0.02^2), 3 steps of N(0,1)
    gradients, zero momentum; trajectories compared directly."""
    wl = W.WORKLOADS["fp32_128x512"]
    T = W.make_muon_tensors(wl, "cpu")
    Wg = T.params[0].clone().to(DEV)
    Mg = T.moms[0].clone().to(DEV)
    Wo = f64(T.params[0])
    Mo = f64(T.moms[0])
    rms = torch.zeros(1, device=DEV)
    for step in range(wl.steps):
        G = W.make_grads(wl, "cpu", step).view(128, 512)
        Gg = G.to(DEV)
        W_prev = f64(Wg)
        mod.muon_step([Wg], [Gg], [Mg], ns_dtype=torch.float32, update_rms=rms, **HYP)
        torch.cuda.synchronize()
        Wo_prev = Wo
        Wo, Mo, Xo, rms_o = mo.muon_step(Wo, f64(G), Mo, abc=mo.NS_COEFFS, **HYP)
        # update of this step, and the whole trajectory so far
        upd_err = sp.rel_fro(W_prev - f64(Wg), Wo_prev - Wo)
        traj_err = np.linalg.norm(f64(Wg) - Wo) / np.linalg.norm(Wo - f64(T.params[0]))
        print(f"step {step}: update {upd_err:.2e} trajectory {traj_err:.2e}")
        assert upd_err <= 1e-4 and traj_err <= 1e-4
        assert sp.rel_fro(f64(Mg), Mo) <= 1e-6
        assert abs(rms.item() - rms_o) <= 1e-4 * rms_o


# ---------------------------------------------------------------- full step, bf16

MIXED = [(300, 700), (700, 300), (64, 2048), (2048, 64), (128, 128), (1, 300),
         (257, 1031), (1031, 257), (300, 700)]


def _mixed_state(seed, shapes, grad_dtype=torch.float32, mom_dtype=torch.bfloat16,
                 zero_mom=False):
    Ps, Gs, Ms = [], [], []
    for i, s in enumerate(shapes):
        Ps.append(randn(s, seed + 3 * i, 0.02))
        Gs.append(randn(s, seed + 3 * i + 1, 1e-3 * (1 + i), grad_dtype))
        Ms.append(torch.zeros(s, device=DEV, dtype=mom_dtype) if zero_mom
                  else randn(s, seed + 3 * i + 2, 1e-3, mom_dtype))
    return Ps, Gs, Ms


def _check_step(P0, G, M0, P1, M1, rms, hyp, ns_bf16=True, mom_bf16=True):
    """Step-local parity of one matrix."""
    Wo, Mo, Xo, rms_o = mo.muon_step(P0, G, M0, abc=mo.NS_COEFFS, **hyp)
    upd_g = P0 - P1
    upd_o = P0 - Wo
    err = sp.rel_fro(upd_g, upd_o)
    if mom_bf16:
        # half a bf16 ulp of the result, plus the fp32 evaluation error of
        # mu*M + G, which matters where the two terms cancel
        tol = np.abs(Mo) * (2.0 ** -8 + 2.0 ** -20) + \
            (np.abs(hyp["mu"] * M0) + np.abs(G)) * 2.0 ** -22 + 1e-30
        assert np.all(np.abs(M1 - Mo) <= tol)
    else:
        assert sp.rel_fro(M1, Mo) <= 1e-6
    r, c = P0.shape
    scale = hyp["rms_scale"] * math.sqrt(max(r, c))
    X_rec = (upd_g - hyp["lr"] * hyp["wd"] * P0) / (hyp["lr"] * scale)
    _, N = mo.momentum_update(M0, G, hyp["mu"], hyp["nesterov"])
    if ns_bf16:
        assert err <= 2e-2, err
        if min(r, c) > 1:
            assert sp.per_sigma_deviation(X_rec, N, hyp["ns_steps"], eps=hyp["eps"]) <= 0.05
        if rms is not None:
            assert abs(rms - rms_o) <= 2e-2 * rms_o
    else:
        assert err <= 1e-4, err
        if rms is not None:
            assert abs(rms - rms_o) <= 1e-4 * rms_o
    return err


@pytest.mark.parametrize("grad_dtype", [torch.float32, torch.bfloat16])
def test_step_bf16_mixed_shapes(mod, grad_dtype):
    Ps, Gs, Ms = _mixed_state(100, MIXED, grad_dtype)
    P0 = [f64(p) for p in Ps]
    M0 = [f64(m) for m in Ms]
    G0 = [f64(g) for g in Gs]
    rms = torch.zeros(len(Ps), device=DEV)
    mod.muon_step(Ps, Gs, Ms, update_rms=rms, **HYP)
    torch.cuda.synchronize()
    for i in range(len(Ps)):
        e = _check_step(P0[i], G0[i], M0[i], f64(Ps[i]), f64(Ms[i]), rms[i].item(), HYP)
        print(MIXED[i], f"update rel_fro {e:.3e}")


def test_step_super_block_order(mod, monkeypatch):
    """64-wide tiles make these matrices 16 and 32 tiles a side, so the Gram,
    polynomial, update and apply products run in the super-block tile order
    used for large matrices, two shape groups per launch."""
    monkeypatch.setenv("MO_TILE", "64")
    shapes = [(1024, 1024), (1024, 2048), (2048, 1024)]
    Ps, Gs, Ms = _mixed_state(700, shapes)
    P0 = [f64(p) for p in Ps]
    M0 = [f64(m) for m in Ms]
    G0 = [f64(g) for g in Gs]
    rms = torch.zeros(len(Ps), device=DEV)
    mod.muon_step(Ps, Gs, Ms, update_rms=rms, **HYP)
    torch.cuda.synchronize()
    for i in range(len(Ps)):
        e = _check_step(P0[i], G0[i], M0[i], f64(Ps[i]), f64(Ms[i]), rms[i].item(), HYP)
        print(shapes[i], f"update rel_fro {e:.3e}")


@pytest.mark.parametrize("waves", ["4", "8"])
def test_step_tile256_waves(mod, monkeypatch, waves):
    """256-wide tiles with 4 or 8 waves per workgroup on every product
    (Gram, polynomial, update, apply), on shapes with ragged edges, both
    orientations and diagonal tiles that straddle several waves."""
    monkeypatch.setenv("MO_TILE", "256")
    monkeypatch.setenv("MO_WAVES", waves)
    shapes = [(300, 700), (700, 300), (512, 1024), (257, 1031), (1031, 257), (64, 600)]
    Ps, Gs, Ms = _mixed_state(800, shapes)
    P0 = [f64(p) for p in Ps]
    M0 = [f64(m) for m in Ms]
    G0 = [f64(g) for g in Gs]
    rms = torch.zeros(len(Ps), device=DEV)
    mod.muon_step(Ps, Gs, Ms, update_rms=rms, **HYP)
    torch.cuda.synchronize()
    for i in range(len(Ps)):
        e = _check_step(P0[i], G0[i], M0[i], f64(Ps[i]), f64(Ms[i]), rms[i].item(), HYP)
        print(shapes[i], waves, f"update rel_fro {e:.3e}")


def test_ns_store_tile256_waves8(mod, monkeypatch):
    """The store epilogue (orthogonalize only) with 8 waves."""
    monkeypatch.setenv("MO_TILE", "256")
    monkeypatch.setenv("MO_WAVES", "8")
    for shape in [(300, 700), (700, 300)]:
        x = randn(shape, 17 + shape[0], dtype=torch.bfloat16)
        X = mod.newton_schulz(x, ns_steps=5)
        torch.cuda.synchronize()
        ref, _ = mo.orthogonalize(f64(x), 5, eps=1e-7)
        assert sp.rel_fro(f64(X), ref) <= 2e-2


@pytest.mark.parametrize("abc", [(1.5, -0.5, 0.0), (3.0, -3.2, 1.2)])
def test_ns_custom_coeffs_tile256(mod, monkeypatch, abc):
    """Other polynomial coefficients on 256-wide tiles: without the quintic
    term (c = 0, which takes the 4-wave polynomial product that reads S in
    its epilogue) and with a different b / c ratio (8 waves, b S folded into
    the accumulators)."""
    monkeypatch.setenv("MO_TILE", "256")
    for shape in [(300, 700), (512, 512)]:
        x = randn(shape, 23 + shape[1], dtype=torch.bfloat16)
        X = mod.newton_schulz(x, ns_steps=5, abc=abc)
        torch.cuda.synchronize()
        ref, _ = mo.orthogonalize(f64(x), 5, abc=abc, eps=1e-7)
        err = sp.rel_fro(f64(X), ref)
        print(shape, abc, f"rel_fro {err:.3e}")
        assert err <= 2e-2


@pytest.mark.parametrize("scaling", ["hidden", "update_norm"])
@pytest.mark.parametrize("ns_steps", [0, 1, 5])
@pytest.mark.parametrize("tile", [None, "256"])
def test_step_alternative_scalings(mod, monkeypatch, scaling, ns_steps, tile):
    """Section 3.1's Eq. 5 (0.2 sqrt(H)) and Eq. 6 (0.2 / RMS(O)) through a
    plan, against the oracle's same scaling; the last matrix has a zero
    gradient and momentum (Eq. 6: decay only)."""
    if tile:
        monkeypatch.setenv("MO_TILE", tile)
    shapes = [(300, 700), (700, 300), (64, 64), (1, 300), (257, 1031), (96, 160)]
    Ps, Gs, Ms = _mixed_state(900 + ns_steps, shapes)
    Gs[-1].zero_()
    Ms[-1].zero_()
    P0 = [f64(p) for p in Ps]
    M0 = [f64(m) for m in Ms]
    G0 = [f64(g) for g in Gs]
    hyp = dict(HYP, ns_steps=ns_steps)
    H = 1024.0
    rms = torch.full((len(Ps),), -1.0, device=DEV)
    plan = mod.MuonPlan(Ps, Gs, Ms)
    plan.step(update_rms=rms, scaling=scaling, hidden=H, **hyp)
    torch.cuda.synchronize()
    plan.close()
    for i, shp in enumerate(shapes):
        Wo, Mo, Xo, rms_o = mo.muon_step(P0[i], G0[i], M0[i], abc=mo.NS_COEFFS, scaling=scaling,
                                         hidden=H, **hyp)
        P1 = f64(Ps[i])
        if i == len(shapes) - 1:
            assert np.allclose(P1, P0[i] * (1 - hyp["lr"] * hyp["wd"]), rtol=1e-6, atol=0)
            assert rms[i].item() == 0.0
            continue
        err = sp.rel_fro(P0[i] - P1, P0[i] - Wo)
        print(shp, scaling, ns_steps, f"update rel_fro {err:.3e}")
        assert err <= 2e-2, (shp, err)
        assert abs(rms[i].item() - rms_o) <= 2e-2 * rms_o
        if scaling == "update_norm":
            upd = (P0[i] - P1) / hyp["lr"] - hyp["wd"] * P0[i]
            assert abs(math.sqrt(np.mean(upd ** 2)) - 0.2) <= 2e-3


@pytest.mark.parametrize("ns_steps", [1, 2, 5])
@pytest.mark.parametrize("scaling", ["shape", "hidden"])
def test_small_matrix_fused_path(mod, ns_steps, scaling):
    """Shape groups of >= 32 matrices with m <= 128 take the fused kernel
    (the iteration carried out on m x m matrices at about fp32 precision,
    then X_N = Q X_0 and the apply, one workgroup per matrix): ragged and
    oriented shapes (m = 128 with n a multiple of 128 in both orientations
    takes the kernel's full-tile W path), sampled matrices against the
    oracle, update RMS of every matrix.  Its error is the bf16 storage of X_0, as in the CPU model
    ``bf16_model.ns_gram_space`` (test_bf16_model.py): off the square shape
    the bounds are that model's figures with a margin (1.6-2.1e-3 Frobenius
    measured at N <= 5), well inside the bf16 bar and at N = 10 below what
    bf16 iterates reach."""
    groups = [((128, 512), 32), ((700, 96), 33), ((100, 300), 34), ((128, 128), 32), ((384, 128), 32)]
    shapes = [s for s, n in groups for _ in range(n)]
    Ps, Gs, Ms = _mixed_state(1300 + ns_steps, shapes)
    P0 = [f64(p) for p in Ps]
    M0 = [f64(m) for m in Ms]
    G0 = [f64(g) for g in Gs]
    hyp = dict(HYP, ns_steps=ns_steps)
    rms = torch.zeros(len(Ps), device=DEV)
    plan = mod.MuonPlan(Ps, Gs, Ms)
    plan.step(update_rms=rms, scaling=scaling, hidden=512.0, **hyp)
    torch.cuda.synchronize()
    plan.close()
    start = 0
    for (shp, n) in groups:
        for i in (start, start + n // 2, start + n - 1):
            Wo, Mo, Xo, rms_o = mo.muon_step(P0[i], G0[i], M0[i], abc=mo.NS_COEFFS, scaling=scaling,
                                             hidden=512.0, **hyp)
            P1, M1 = f64(Ps[i]), f64(Ms[i])
            err = sp.rel_fro(P0[i] - P1, P0[i] - Wo)
            r, cc = shp
            sq = r == cc
            scale = 0.2 * (math.sqrt(512.0) if scaling == "hidden" else math.sqrt(max(r, cc)))
            X_rec = (P0[i] - P1 - 1e-3 * 0.1 * P0[i]) / (1e-3 * scale)
            _, N = mo.momentum_update(M0[i], G0[i], 0.95, True)
            dev = sp.per_sigma_deviation(X_rec, N, ns_steps, eps=1e-7)
            print(shp, ns_steps, scaling, f"update rel_fro {err:.3e}, per-sigma {dev:.4f}")
            if sq:
                # a square matrix's smallest singular values are tiny and
                # vary from matrix to matrix; the m x m recursion amplifies
                # their rounding as bf16 iterates do (per-sigma 0.015 on one
                # [128, 128] matrix at N = 5): the bf16 bars
                assert err <= 1e-2, (shp, i, err)
                assert dev <= 0.05, (shp, i, dev)
            else:
                assert err <= 4e-3, (shp, i, err)
                assert dev <= 0.002, (shp, i, dev)
            tol = np.abs(Mo) * (2.0 ** -8 + 2.0 ** -20) + (np.abs(0.95 * M0[i]) + np.abs(G0[i])) * 2.0 ** -22 + 1e-30
            assert np.all(np.abs(M1 - Mo) <= tol)
            assert abs(rms[i].item() - rms_o) <= 2e-2 * rms_o
        start += n


def test_small_fused_edge_shapes(mod):
    """Fused small-matrix kernel on the edges of its domain: one-row and
    one-column matrices, a 5 x 7 matrix (both sides far below one 128
    panel), and zero gradients with zero momentum in the middle of a group
    (X_N = 0: a decay-only step and an update RMS of 0)."""
    groups = [((1, 300), 32), ((300, 1), 32), ((5, 7), 32), ((64, 200), 33)]
    shapes = [s for s, n in groups for _ in range(n)]
    Ps, Gs, Ms = _mixed_state(1600, shapes)
    zero = [len(shapes) - 10, len(shapes) - 9]
    for i in zero:
        Gs[i].zero_()
        Ms[i].zero_()
    P0 = [f64(p) for p in Ps]
    M0 = [f64(m) for m in Ms]
    G0 = [f64(g) for g in Gs]
    rms = torch.zeros(len(shapes), device=DEV)
    plan = mod.MuonPlan(Ps, Gs, Ms)
    plan.step(update_rms=rms, **HYP)
    torch.cuda.synchronize()
    plan.close()
    for i in [0, 31, 32, 63, 64, 95, 96, len(shapes) - 1] + zero:
        P1 = f64(Ps[i])
        if i in zero:
            assert np.allclose(P1, P0[i] * (1 - HYP["lr"] * HYP["wd"]), rtol=1e-6, atol=0)
            assert rms[i].item() == 0.0
            continue
        Wo, Mo, Xo, rms_o = mo.muon_step(P0[i], G0[i], M0[i], abc=mo.NS_COEFFS, **HYP)
        err = sp.rel_fro(P0[i] - P1, P0[i] - Wo)
        print(shapes[i], f"update rel_fro {err:.3e}")
        assert err <= 4e-3, (shapes[i], i, err)
        assert abs(rms[i].item() - rms_o) <= 2e-2 * rms_o


@pytest.mark.parametrize("abc,steps", [((1.5, -0.5, 0.0), 3), ((2.0, -1.5, 0.5), 4)])
def test_small_fused_custom_coefficients(mod, abc, steps):
    """Custom Eq. 2 coefficients through the fused kernel: the cubic
    (c = 0, P = a I + b S) and another quintic, against the oracle with
    the same coefficients, off the default five steps."""
    shapes = [(100, 300)] * 33 + [(256, 64)] * 32
    Ps, Gs, Ms = _mixed_state(1700, shapes)
    P0 = [f64(p) for p in Ps]
    M0 = [f64(m) for m in Ms]
    G0 = [f64(g) for g in Gs]
    hyp = dict(HYP, ns_steps=steps)
    mod.muon_step(Ps, Gs, Ms, abc=abc, **hyp)
    torch.cuda.synchronize()
    for i in (0, 32, 33, len(shapes) - 1):
        Wo, Mo, Xo, rms_o = mo.muon_step(P0[i], G0[i], M0[i], abc=abc, **hyp)
        err = sp.rel_fro(P0[i] - f64(Ps[i]), P0[i] - Wo)
        print(shapes[i], abc, steps, f"update rel_fro {err:.3e}")
        assert err <= 4e-3, (shapes[i], abc, err)


def test_small_fused_ill_conditioned(mod, monkeypatch):
    """Gram-space kernel on inputs where the m x m recursion is most
    sensitive: rank-deficient gradients (rank 16 of 128) and spectra spread
    over six decades, N = 5, zero momentum.  The fused kernel stays finite
    and at least as close to the oracle as the bf16 iterates of the general
    kernels (MO_NO_SMALL=1) on the same step -- the CPU model's finding in
    test_bf16_model.py, here on the GPU."""
    g = torch.Generator().manual_seed(1900)

    def spectrum_matrix(m, n, sig):
        U, _ = torch.linalg.qr(torch.randn(m, m, generator=g, dtype=torch.float64))
        V, _ = torch.linalg.qr(torch.randn(n, m, generator=g, dtype=torch.float64))
        return (U * torch.as_tensor(sig)) @ V.T

    shapes, grads = [], []
    for i in range(32):
        sig = np.r_[np.ones(16), np.zeros(112)] * 1e-3
        grads.append(spectrum_matrix(128, 512, sig))
        shapes.append((128, 512))
    for i in range(32):
        grads.append(spectrum_matrix(128, 2048, np.logspace(0, -6, 128) * 1e-3))
        shapes.append((128, 2048))
    P_init = [torch.randn(s, generator=g).mul(0.02).to(DEV) for s in shapes]
    outs = {}
    for off in ("0", "1"):
        monkeypatch.setenv("MO_NO_SMALL", off)
        Ps = [p.clone() for p in P_init]
        Gs = [x.float().to(DEV) for x in grads]
        Ms = [torch.zeros(s, device=DEV, dtype=torch.bfloat16) for s in shapes]
        mod.muon_step(Ps, Gs, Ms, **HYP)
        torch.cuda.synchronize()
        outs[off] = [f64(p) for p in Ps]
    P0 = [f64(p) for p in P_init]
    for i in (0, 31, 32, 63):
        assert np.all(np.isfinite(outs["0"][i]))
        G0 = f64(grads[i].float())
        Wo, Mo, Xo, rms_o = mo.muon_step(P0[i], G0, np.zeros(shapes[i]), abc=mo.NS_COEFFS, **HYP)
        e_fused = sp.rel_fro(P0[i] - outs["0"][i], P0[i] - Wo)
        e_general = sp.rel_fro(P0[i] - outs["1"][i], P0[i] - Wo)
        print(shapes[i], f"fused {e_fused:.3e}, general {e_general:.3e}")
        assert e_fused <= e_general, (i, e_fused, e_general)


def test_small_group_beyond_five_steps_takes_general_kernels(mod, monkeypatch):
    """N = 10 on groups that would otherwise take the fused kernel: the
    Gram-space recursion is not used past 5 steps (rounding can turn a tiny
    direction's Gram eigenvalue negative, and the polynomial grows it
    without bound), so the per-product kernels run and the bf16 N = 10
    figures apply: per-sigma <= 0.05 and Frobenius well inside 4e-2 on
    rectangular shapes.  Their bitwise equality with MO_NO_SMALL=1 shows
    that the fused kernel was not used."""
    groups = [((128, 512), 32), ((700, 96), 33)]
    shapes = [s for s, n in groups for _ in range(n)]
    outs = []
    for off in ("0", "1"):
        monkeypatch.setenv("MO_NO_SMALL", off)
        Ps, Gs, Ms = _mixed_state(1500, shapes)
        P0 = [f64(p) for p in Ps]
        M0 = [f64(m) for m in Ms]
        G0 = [f64(g) for g in Gs]
        mod.muon_step(Ps, Gs, Ms, **dict(HYP, ns_steps=10))
        torch.cuda.synchronize()
        outs.append([f64(p) for p in Ps])
    for a, b in zip(outs[0], outs[1]):
        assert np.array_equal(a, b)
    for i in (0, 31, 32, len(shapes) - 1):
        Wo, Mo, Xo, rms_o = mo.muon_step(P0[i], G0[i], M0[i], abc=mo.NS_COEFFS, **dict(HYP, ns_steps=10))
        err = sp.rel_fro(P0[i] - outs[0][i], P0[i] - Wo)
        r, cc = shapes[i]
        X_rec = (P0[i] - outs[0][i] - 1e-3 * 0.1 * P0[i]) / (1e-3 * 0.2 * math.sqrt(max(r, cc)))
        _, N = mo.momentum_update(M0[i], G0[i], 0.95, True)
        dev = sp.per_sigma_deviation(X_rec, N, 10, eps=1e-7)
        print(shapes[i], f"N = 10 update rel_fro {err:.3e}, per-sigma {dev:.4f}")
        assert err <= 4e-2 and dev <= 0.05, (shapes[i], err, dev)


def test_small_fused_matches_general_path(mod, monkeypatch):
    """The fused kernel (Gram-space iteration, about fp32 precision) and the
    per-product kernels (bf16 iterates) agree on the same step to within the
    bf16 path's own error (~8e-3 against the oracle at this shape, N = 5)."""
    shapes = [(128, 2048)] * 40
    outs = []
    for off in ("0", "1"):
        monkeypatch.setenv("MO_NO_SMALL", off)
        Ps, Gs, Ms = _mixed_state(1400, shapes)
        mod.muon_step(Ps, Gs, Ms, **HYP)
        torch.cuda.synchronize()
        outs.append([f64(p) for p in Ps])
    P0 = f64(_mixed_state(1400, shapes)[0][0])
    for a, b in zip(outs[0][:5], outs[1][:5]):
        assert sp.rel_fro(P0 - a, P0 - b) <= 1e-2


def test_plan_scaling_validation(mod):
    x = [randn((64, 128), 1)]
    plan = mod.MuonPlan(x, [randn((64, 128), 2)], [torch.zeros(64, 128, device=DEV, dtype=torch.bfloat16)])
    with pytest.raises(ValueError):
        plan.step(lr=1e-3, scaling="hidden")          # H missing
    with pytest.raises(mod.MuonError):
        plan.step(lr=1e-3, scaling="hidden", hidden=0.5)
    plan.close()


@pytest.mark.parametrize("variant", [{"nesterov": False}, {"ns_steps": 0}, {"ns_steps": 1},
                                     {"ns_steps": 10}, {"mu": 0.0}])
def test_step_variants(mod, variant):
    shapes = [(200, 456), (456, 200), (64, 64)]
    if variant.get("ns_steps") == 10:
        shapes = [(200, 456), (456, 200), (96, 300), (64, 64)]
    Ps, Gs, Ms = _mixed_state(200, shapes)
    P0, G0, M0 = [f64(p) for p in Ps], [f64(g) for g in Gs], [f64(m) for m in Ms]
    hyp = dict(HYP, **variant)
    rms = torch.zeros(len(Ps), device=DEV)
    mod.muon_step(Ps, Gs, Ms, update_rms=rms, **hyp)
    torch.cuda.synchronize()
    for i in range(len(Ps)):
        if hyp["ns_steps"] == 10:
            # bf16 iterates at N=10 can exceed 2e-2 Frobenius (the slope of
            # the 10-fold map reaches ~86); gate on the per-sigma criterion
            Wo, Mo, Xo, rms_o = mo.muon_step(P0[i], G0[i], M0[i], abc=mo.NS_COEFFS, **hyp)
            r, c = shapes[i]
            X_rec = (P0[i] - f64(Ps[i]) - hyp["lr"] * hyp["wd"] * P0[i]) / (
                hyp["lr"] * hyp["rms_scale"] * math.sqrt(max(r, c)))
            _, N = mo.momentum_update(M0[i], G0[i], hyp["mu"], hyp["nesterov"])
            dev = sp.per_sigma_deviation(X_rec, N, 10, eps=hyp["eps"])
            fro = sp.rel_fro(P0[i] - f64(Ps[i]), P0[i] - Wo)
            print(f"N = 10 {shapes[i]}: per-sigma {dev:.3e}, update rel_fro {fro:.3e}")
            # measured on the GPU: per-sigma 0.012-0.039 (square 0.012),
            # rel_fro 1.7-1.8e-2; bf16 at N = 10 is held to the per-sigma
            # gate, and its Frobenius error is reported with a 4e-2 bound
            assert dev <= 0.05
            assert fro <= 4e-2
        else:
            _check_step(P0[i], G0[i], M0[i], f64(Ps[i]), f64(Ms[i]), rms[i].item(), hyp)


def test_zero_gradient_is_decay_only(mod):
    shapes = [(130, 260), (260, 130)]
    Ps = [randn(s, 300 + i, 0.02) for i, s in enumerate(shapes)]
    Gs = [torch.zeros(s, device=DEV) for s in shapes]
    Ms = [torch.zeros(s, device=DEV, dtype=torch.bfloat16) for s in shapes]
    P0 = [p.clone() for p in Ps]
    rms = torch.full((2,), -1.0, device=DEV)
    mod.muon_step(Ps, Gs, Ms, update_rms=rms, **HYP)
    torch.cuda.synchronize()
    for p0, p1, m in zip(P0, Ps, Ms):
        exp = f64(p0) - HYP["lr"] * HYP["wd"] * f64(p0)
        assert np.all(np.abs(f64(p1) - exp) <= np.abs(exp) * 2.0 ** -23)
        assert torch.count_nonzero(m).item() == 0
    assert torch.all(rms == 0).item()


def test_fp32_path_mixed_shapes(mod):
    shapes = [(100, 300), (300, 100), (64, 64), (1, 77), (129, 200)]
    Ps, Gs, Ms = _mixed_state(400, shapes, torch.float32, torch.float32)
    P0, G0, M0 = [f64(p) for p in Ps], [f64(g) for g in Gs], [f64(m) for m in Ms]
    rms = torch.zeros(len(Ps), device=DEV)
    mod.muon_step(Ps, Gs, Ms, ns_dtype=torch.float32, update_rms=rms, **HYP)
    torch.cuda.synchronize()
    for i in range(len(Ps)):
        _check_step(P0[i], G0[i], M0[i], f64(Ps[i]), f64(Ms[i]), rms[i].item(), HYP,
                    ns_bf16=False, mom_bf16=False)


# ---------------------------------------------------------------- execution properties

def _run_once(mod, shapes, seed, **kw):
    Ps, Gs, Ms = _mixed_state(seed, shapes)
    mod.muon_step(Ps, Gs, Ms, **HYP, **kw)
    torch.cuda.synchronize()
    return Ps, Ms


def test_deterministic_and_chunking_and_plan(mod):
    # the 33 [128, 384] matrices take the fused small-matrix kernel, in one
    # launch with the full workspace and one matrix at a time with the least
    shapes = [(256, 512)] * 5 + [(512, 256)] * 3 + [(64, 1000)] * 2 + [(128, 384)] * 33
    Pa, Ma = _run_once(mod, shapes, 500)
    Pb, Mb = _run_once(mod, shapes, 500)
    for x, y in zip(Pa + Ma, Pb + Mb):
        assert torch.equal(x, y)
    # smallest workspace: every shape group runs in several passes
    full, mn = mod.muon_workspace_size(shapes)
    ws = torch.empty(mn, dtype=torch.uint8, device=DEV)
    Pc, Mc = _run_once(mod, shapes, 500, workspace=ws)
    for x, y in zip(Pa + Ma, Pc + Mc):
        assert torch.equal(x, y)
    # the plan entry point
    Ps, Gs, Ms = _mixed_state(500, shapes)
    plan = mod.MuonPlan(Ps, Gs, Ms)
    plan.step(**HYP)
    torch.cuda.synchronize()
    for x, y in zip(Pa + Ma, Ps + Ms):
        assert torch.equal(x, y)
    plan.close()


def test_resume_equivalence(mod):
    """3 steps straight vs 2 steps, a host round trip of all state, 1 step."""
    shapes = [(192, 320), (320, 192)]
    def run(split):
        Ps, _, Ms = _mixed_state(600, shapes, zero_mom=True)
        for step in range(3):
            Gs = [randn(s, 700 + 10 * step + i, 1e-3) for i, s in enumerate(shapes)]
            mod.muon_step(Ps, Gs, Ms, **HYP)
            if split and step == 1:
                torch.cuda.synchronize()
                Ps = [p.cpu().to(DEV) for p in Ps]
                Ms = [m.cpu().to(DEV) for m in Ms]
        torch.cuda.synchronize()
        return Ps + Ms
    for x, y in zip(run(False), run(True)):
        assert torch.equal(x, y)


# ---------------------------------------------------------------- AdamW

def _adamw_close(p0, p1, Wo):
    """fp32 AdamW against fp64: 1e-5 relative on the update, plus the fp32
    rounding of the stored weight (one ulp of |W|)."""
    err = np.abs(p1 - Wo)
    tol = 1e-5 * np.abs(p0 - Wo) + np.abs(Wo) * 2.0 ** -23 + 1e-30
    assert np.all(err <= tol), float(np.max(err / tol))


@pytest.mark.parametrize("grad_dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("t", [1, 5])
def test_adamw(mod, grad_dtype, t):
    sizes = [1, 3, 1536, 2049, 4096 * 3 + 5, 65536]
    Ps = [randn((n,), 800 + i, 0.02) for i, n in enumerate(sizes)]
    Gs = [randn((n,), 900 + i, 1e-3, grad_dtype) for i, n in enumerate(sizes)]
    ms = [randn((n,), 1000 + i, 1e-4) if t > 1 else torch.zeros(n, device=DEV)
          for i, n in enumerate(sizes)]
    vs = [randn((n,), 1100 + i, 1e-4).square() if t > 1 else torch.zeros(n, device=DEV)
          for i, n in enumerate(sizes)]
    before = [(f64(p), f64(g), f64(m), f64(v)) for p, g, m, v in zip(Ps, Gs, ms, vs)]
    mod.adamw_step(Ps, Gs, ms, vs, lr=1e-3, wd=0.1, step=t)
    torch.cuda.synchronize()
    for (p0, g0, m0, v0), p1, m1, v1 in zip(before, Ps, ms, vs):
        Wo, mo_, vo = mo.adamw_step(p0, g0, m0, v0, lr=1e-3, wd=0.1, t=t)
        _adamw_close(p0, f64(p1), Wo)
        assert sp.rel_fro(f64(m1), mo_) <= 1e-6
        assert sp.rel_fro(f64(v1), vo) <= 1e-6


def test_optimizer_front(mod):
    """MuonAdamW routes matrices to Muon and the rest to AdamW."""
    mats = [torch.nn.Parameter(randn((96, 160), 1200 + i, 0.02)) for i in range(3)]
    vecs = [torch.nn.Parameter(torch.ones(96, device=DEV))]
    for p in mats + vecs:
        p.grad = torch.randn_like(p) * 1e-3
    before = [f64(p) for p in mats + vecs]
    grads = [f64(p.grad) for p in mats + vecs]
    opt = mod.MuonAdamW(mats, vecs, lr=1e-3, wd=0.1)
    opt.step()
    torch.cuda.synchronize()
    for i in range(3):
        Wo, _, _, _ = mo.muon_step(before[i], grads[i], np.zeros_like(before[i]),
                                   abc=mo.NS_COEFFS, **HYP)
        assert sp.rel_fro(before[i] - f64(mats[i]), before[i] - Wo) <= 2e-2
    z = np.zeros_like(before[3])
    Wo, _, _ = mo.adamw_step(before[3], grads[3], z, z, lr=1e-3, wd=0.1, t=1)
    _adamw_close(before[3], f64(vecs[0]), Wo)


def test_steps_on_two_streams_use_separate_workspaces(mod):
    """Two independent steps queued on two streams through the binding's
    implicit workspaces (cached per device and stream) give the same bits as
    the same steps run one after the other on one stream."""
    shapes_a = [(300, 700), (1031, 257)]
    shapes_b = [(512, 1536), (128, 128)]
    ref = []
    for seed, shapes in ((700, shapes_a), (800, shapes_b)):
        Ps, Gs, Ms = _mixed_state(seed, shapes)
        mod.muon_step(Ps, Gs, Ms, **HYP)
        ref.append((Ps, Ms))
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()     # default priority
    A = _mixed_state(700, shapes_a)
    B = _mixed_state(800, shapes_b)
    torch.cuda.synchronize()
    for _ in range(3):                                     # fresh state each round
        Pa, Ga, Ma = [x.clone() for x in A[0]], A[1], [x.clone() for x in A[2]]
        Pb, Gb, Mb = [x.clone() for x in B[0]], B[1], [x.clone() for x in B[2]]
        torch.cuda.synchronize()
        mod.muon_step(Pa, Ga, Ma, stream=s1, **HYP)
        mod.muon_step(Pb, Gb, Mb, stream=s2, **HYP)
        torch.cuda.synchronize()
        for got, want in zip(Pa + Ma + Pb + Mb, ref[0][0] + ref[0][1] + ref[1][0] + ref[1][1]):
            assert torch.equal(got, want)




RAGGED_SHAPES = [(1408, 2048), (2048, 1408), (300, 700), (700, 300), (640, 900), (384, 1024)]


@pytest.mark.parametrize("variant", [{}, {"ns_steps": 0}, {"ns_steps": 1}, {"waves": "4"}, {"c0": True},
                                     {"scaling": "update_norm"}])
def test_half_empty_last_panel(mod, monkeypatch, variant):
    """Short sides that fill only half of their last 256-row panel (the MoE
    experts' 1408 = 5.5 x 256; 300, 640, 384), both orientations, through a
    plan: 4 waves, no quintic term (the polynomial reading S in its
    epilogue), the update-norm scaling (the RMS-only pass), N = 0 and 1.
    Each matrix against the oracle: update, momentum, update RMS, and the
    per-singular-value deviation at N = 5."""
    if variant.get("waves"):
        monkeypatch.setenv("MO_WAVES", variant["waves"])
    hyp = dict(HYP, ns_steps=variant.get("ns_steps", 5))
    abc = (1.5, -0.5, 0.0) if variant.get("c0") else None
    scaling = variant.get("scaling", "shape")
    Ps, Gs, Ms = _mixed_state(1500, RAGGED_SHAPES)
    P0, G0, M0 = [f64(p) for p in Ps], [f64(g) for g in Gs], [f64(m) for m in Ms]
    rms = torch.full((len(Ps),), -1.0, device=DEV)
    plan = mod.MuonPlan(Ps, Gs, Ms)
    plan.step(update_rms=rms, scaling=scaling, abc=abc, **hyp)
    torch.cuda.synchronize()
    plan.close()
    for i, s in enumerate(RAGGED_SHAPES):
        Wo, Mo, Xo, rms_o = mo.muon_step(P0[i], G0[i], M0[i], abc=abc or mo.NS_COEFFS, scaling=scaling, **hyp)
        err = sp.rel_fro(P0[i] - f64(Ps[i]), P0[i] - Wo)
        print(s, variant, f"update rel_fro {err:.3e}")
        assert err <= 2e-2, (s, err)
        tol = np.abs(Mo) * (2.0 ** -8 + 2.0 ** -20) + (np.abs(0.95 * M0[i]) + np.abs(G0[i])) * 2.0 ** -22 + 1e-30
        assert np.all(np.abs(f64(Ms[i]) - Mo) <= tol)
        assert abs(rms[i].item() - rms_o) <= 2e-2 * rms_o
        if hyp["ns_steps"] == 5 and abc is None and scaling == "shape":
            r, c = s
            X_rec = (P0[i] - f64(Ps[i]) - hyp["lr"] * hyp["wd"] * P0[i]) / (hyp["lr"] * 0.2 * math.sqrt(max(r, c)))
            _, N = mo.momentum_update(M0[i], G0[i], 0.95, True)
            assert sp.per_sigma_deviation(X_rec, N, 5, eps=1e-7) <= 0.05
