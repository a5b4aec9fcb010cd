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
