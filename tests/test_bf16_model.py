"""The bf16 tolerance statements, reproduced by the CPU rounding model
(``tests/bf16_model.py``) on the very inputs of the GPU parity tests.

The pages run Newton-Schulz in bf16 ("Muon is Scalable for LLM Training",
section 2.3) and fix no error budget; the parity bars are 2e-2 relative
Frobenius and 0.05 per singular value.  Where a GPU test allows more, or
gates a case on one criterion only, the figure comes from rounding every
stored iterate to bf16 -- not from the kernels -- and this model shows it:

* [33, 1000] at N = 5: ~2.5e-2 Frobenius (the GPU test's bound is 3e-2);
* N = 10 (the 5-vs-10 comparison of section 2.2): 1.7-1.8e-2 Frobenius on
  the step-variant shapes, below the reported 4e-2 bound, per-sigma <= 0.05;
* square matrices at N = 10: the one to three directions whose normalised
  singular value lies below ~2^-8 / sqrt(m) (where a bf16 rounding of the
  first iterates, ~2^-9 / sqrt(m) per direction, is comparable to the
  direction itself) are lifted by ~a^10 into the steepest part of the
  10-fold map, so their per-sigma deviation reaches 0.12-0.17, while every
  direction above that stays within 0.065 (up to 0.06 where the 10-fold
  map's slope, up to ~86, amplifies rounding) -- the reading behind the
  large-matrix test's square-shape gate at N = 10;
* the large-matrix workload at N = 10 (opt-in: 4 minutes of CPU, set
  MO_FULL_SIZE_MODEL=1): on a Gaussian [8192, 8192] the model gives
  2.15e-2 Frobenius, 0.040 per-sigma above the floor and 0.074 in all; on
  a Gaussian [8192, 28672] 2.19e-2 and 0.052, the worst directions at
  x0 ~ 0.0123 -- the GPU measures 2.19e-2 / 0.040 / 0.16 and 2.15e-2 /
  0.051 on the workload's own matrices, so these are properties of bf16
  iterates, not of the kernels;
* the model itself, with rounding switched off, agrees with the fp64
  oracle to fp32 accuracy, and its N = 5 errors on the workload shapes
  are ~0.8-0.9e-2, matching the GPU's.

The fused small-matrix path (groups of m <= 128 matrices) does not form
bf16 iterates: it iterates on the m x m Gram matrix with split-bf16
products (``bf16_model.ns_gram_space``).  Its tests below pin that model to
the oracle on exact inputs, give its error on Gaussian inputs (the bf16
storage of X_0, ~1.7-2.1e-3) and show why the path stops at N = 5.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import bf16_model as bm
from oracle import muon_oracle as mo, spectral as sp


def _randn(shape, seed, std=1.0, dtype=torch.float32):
    """The GPU parity tests' input generator (torch CPU generator)."""
    g = torch.Generator()
    g.manual_seed(seed)
    return (torch.randn(*shape, generator=g) * std).to(dtype).double().numpy()


def test_model_without_rounding_is_the_iteration():
    for shape in [(96, 300), (300, 96), (64, 64)]:
        x = _randn(shape, 5 + shape[0])
        for steps in (0, 1, 5, 10):
            ref, _ = mo.orthogonalize(x, steps)
            assert sp.rel_fro(bm.ns_bf16(x, steps, rounding=False), ref) <= 2e-5


def test_to_bf16_rounds_to_nearest_even():
    x = np.array([1.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -7 + 2.0 ** -9, -3.14159],
                 dtype=np.float32)
    got = bm.to_bf16(x)
    # ties to even: 1 + 2^-8 -> 1; 1 + 3 * 2^-8 -> 1 + 2^-6
    assert got[0] == 1.0 and got[1] == 1.0 and got[2] == np.float32(1.0 + 2.0 ** -6)
    assert got[3] == np.float32(1.0 + 2.0 ** -7)        # 1.25 ulp: down
    assert got[4] == np.float32(-3.140625)


def test_thin_33x1000_is_near_2p5e_2():
    x = _randn((33, 1000), 11 + 33 + 7000, dtype=torch.bfloat16)
    ref, _ = mo.orthogonalize(x, 5)
    X = bm.ns_bf16(x, 5)
    e = sp.rel_fro(X, ref)
    assert 2.2e-2 <= e <= 2.8e-2, e
    assert sp.per_sigma_deviation(X, x, 5) <= 0.05


@pytest.mark.parametrize("shape", [(128, 512), (300, 700), (1536, 1536), (64, 2048), (257, 1031)])
def test_n5_workload_like_shapes_stay_near_1e_2(shape):
    x = _randn(shape, 11 + shape[0] + 7 * shape[1], dtype=torch.bfloat16)
    ref, _ = mo.orthogonalize(x, 5)
    X = bm.ns_bf16(x, 5)
    assert sp.rel_fro(X, ref) <= 1.2e-2
    assert sp.per_sigma_deviation(X, x, 5) <= 0.011


def test_n10_step_variant_shapes():
    """The inputs of test_parity_gpu.py::test_step_variants at N = 10."""
    shapes = [(200, 456), (456, 200), (96, 300), (64, 64)]
    for i, s in enumerate(shapes):
        G = _randn(s, 200 + 3 * i + 1, 1e-3 * (1 + i))
        M = _randn(s, 200 + 3 * i + 2, 1e-3, torch.bfloat16)
        N = bm.nesterov_input_fp32(M, G)
        ref, _ = mo.orthogonalize(N, 10)
        X = bm.ns_bf16(N, 10)
        e = sp.rel_fro(X, ref)
        assert 1.2e-2 <= e <= 2.5e-2, (s, e)
        assert sp.per_sigma_deviation(X, N, 10) <= 0.05, s


def resolved_floor(m: int) -> float:
    """Normalised singular value below which bf16 iterates cannot follow a
    direction at N = 10 (about twice the per-direction rounding noise of
    an iterate of a short side m)."""
    return 2.0 ** -8 / np.sqrt(m)


@pytest.mark.parametrize("m", [128, 256, 512])
def test_square_n10_deviation_sits_in_tiny_directions(m):
    worst_all, worst_resolved = 0.0, 0.0
    for seed in (1, 2, 3):
        x = np.random.default_rng(seed).standard_normal((m, m))
        ref, _ = mo.orthogonalize(x, 10)
        X = bm.ns_bf16(x, 10)
        assert sp.rel_fro(X, ref) <= 2.6e-2
        sig, proj = sp.per_sigma_projections_gram(X, x)
        x0 = sig / np.sqrt(np.sum(x * x))
        dev = np.abs(proj - sp.scalar_map(x0, 10))
        worst_all = max(worst_all, float(dev.max()))
        worst_resolved = max(worst_resolved, float(dev[x0 >= resolved_floor(m)].max()))
        # at N = 5 the same inputs stay far inside the bar
        X5 = bm.ns_bf16(x, 5)
        assert sp.per_sigma_deviation_gram(X5, x, 5) <= 0.01
    assert worst_all >= 0.1               # the tiny directions do not track
    assert worst_resolved <= 0.065        # the rest stays near the 0.05 bar


@pytest.mark.skipif(not __import__("os").environ.get("MO_FULL_SIZE_MODEL"),
                    reason="about 4 minutes of CPU and 12 GB; set MO_FULL_SIZE_MODEL=1")
@pytest.mark.parametrize("shape", [(8192, 8192), (8192, 28672)])
def test_full_size_n10_figures(shape):
    m = min(shape)
    x = np.random.default_rng(1).standard_normal(shape).astype(np.float32).astype(np.float64)
    eig = sp.short_side_eig(x)
    X = bm.ns_bf16(x, 10)
    e = sp.rel_fro(X, sp.ns_closed_form_gram(x, 10, eig=eig))
    sig, proj = sp.per_sigma_projections_gram(X, x, eig)
    x0 = sig / np.sqrt(np.sum(x * x))
    dev = np.abs(proj - sp.scalar_map(x0, 10))
    resolved = float(dev[x0 >= resolved_floor(m)].max())
    print(f"{shape}: rel_fro {e:.3e}, per-sigma {dev.max():.4f}, above the floor {resolved:.4f}, "
          f"worst at x0 {x0[dev.argmax()]:.4f}")
    assert 2.0e-2 <= e <= 2.5e-2
    assert 0.035 <= resolved <= 0.06


# ---- the fused small-matrix path (m <= 128): iteration in Gram space

@pytest.mark.parametrize("shape", [(96, 300), (300, 96), (128, 2048), (17, 40), (128, 128)])
def test_gram_space_model_on_exact_inputs(shape):
    """With a bf16-representable input (X_0 = N exactly) only the split
    products round: the Gram-space recursion reproduces the iteration to
    ~1e-5 (a wrong recursion -- S_{k+1} = P S, a dropped r -- is off by
    O(1), next test).  The square shape's smallest directions make it the
    worst case (3e-4 at N = 5)."""
    x = bm.to_bf16(_randn(shape, 3 + shape[0]).astype(np.float32)).astype(np.float64)
    for steps in (1, 2, 3, 5):
        ref, _ = mo.orthogonalize(x, steps)
        bound = 1e-4 if shape != (128, 128) else (1e-4 if steps <= 2 else 1e-3)
        assert sp.rel_fro(bm.ns_gram_space(x, steps), ref) <= bound, (shape, steps)


def test_gram_space_model_wrong_recursions_fail():
    x = bm.to_bf16(_randn((96, 300), 99).astype(np.float32)).astype(np.float64)
    ref, _ = mo.orthogonalize(x, 5)
    a, b, c = mo.NS_COEFFS
    r = 1.0 / np.sqrt(np.sum(x * x))
    S = r * r * (x @ x.T)
    eye = np.eye(96)
    Q1, Q2, S1, S2 = eye, eye, S.copy(), S.copy()
    for _ in range(5):
        P1 = a * eye + b * S1 + c * S1 @ S1
        S1, Q1 = P1 @ S1, P1 @ Q1              # S_{k+1} = P S: one factor of P dropped
        P2 = a * eye + b * S2 + c * S2 @ S2
        S2, Q2 = P2 @ S2 @ P2, P2 @ Q2
    assert sp.rel_fro(r * Q2 @ x, ref) <= 1e-9            # the exact recursion
    assert sp.rel_fro(r * Q1 @ x, ref) >= 0.1
    assert sp.rel_fro(Q2 @ x, ref) >= 0.1                 # r not applied to X_0


@pytest.mark.parametrize("shape", [(128, 2048), (2048, 128), (128, 512), (700, 96), (100, 300), (96, 300),
                                   (128, 128)])
def test_gram_space_model_accuracy(shape):
    """On Gaussian inputs the Gram-space path's error is the bf16 storage
    of X_0 (~1.7e-3), 3-5x below the bf16 iterates of the general path at
    N = 5: at most 2.1e-3 Frobenius off the square shape (3.2e-3 on
    [128, 128]); per-sigma at most 7e-4 (0.0045 on the square shape)."""
    x = _randn(shape, 11 + shape[1])
    sq = shape[0] == shape[1]
    for steps in (1, 2, 5):
        ref, _ = mo.orthogonalize(x, steps)
        X = bm.ns_gram_space(x, steps)
        fro, dev = sp.rel_fro(X, ref), sp.per_sigma_deviation(X, x, steps)
        assert fro <= (3.5e-3 if sq else 2.5e-3), (shape, steps, fro)
        assert dev <= (0.005 if sq else 0.001), (shape, steps, dev)
        if steps == 5:
            assert fro <= 0.5 * sp.rel_fro(bm.ns_bf16(x, steps), ref)


def _spectrum_matrix(m, n, sig, seed):
    rng = np.random.default_rng(seed)
    U, _ = np.linalg.qr(rng.standard_normal((m, m)))
    V, _ = np.linalg.qr(rng.standard_normal((n, m)))
    return (U * sig) @ V.T


@pytest.mark.parametrize("kind", ["rank half", "logspace 1..1e-6"])
def test_gram_space_is_safe_to_five_steps_only(kind):
    """Why the fused small-matrix path stops at N = 5.  On inputs with
    (near-)zero singular values the Gram-space recursion's rounding can
    make a tiny direction's eigenvalue of S negative; S -> P S P then grows
    it by about a^2 per step with nothing to bound it (the odd polynomial
    bounds singular values, not negative eigenvalues).  Up to N = 6 the
    Gram-space error stays at or below that of bf16 iterates on such
    inputs; at N = 8 it is orders of magnitude larger (bf16 iterates stay
    bounded)."""
    m, n = 128, 2048
    sig = np.r_[np.ones(m // 2), np.zeros(m - m // 2)] if kind == "rank half" else np.logspace(0, -6, m)
    x = _spectrum_matrix(m, n, sig, 5)
    for steps in (3, 5, 6):
        ref, _ = mo.orthogonalize(x, steps)
        assert sp.rel_fro(bm.ns_gram_space(x, steps), ref) <= sp.rel_fro(bm.ns_bf16(x, steps), ref)
    ref, _ = mo.orthogonalize(x, 8)
    with np.errstate(over="ignore", invalid="ignore"):
        gram = sp.rel_fro(bm.ns_gram_space(x, 8), ref)
    bf16 = sp.rel_fro(bm.ns_bf16(x, 8), ref)
    assert bf16 < 2.0
    assert not np.isfinite(gram) or gram > 10.0 * bf16
