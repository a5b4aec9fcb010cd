"""Pins of the per-singular-value parity metric and of the Gram-eigen route.

``spectral.per_sigma_deviation`` is the bf16 gate of every GPU parity test:
``max_i |u_i^T X v_i - f^N(sigma_i / ||N||_F)|`` with ``(u_i, sigma_i, v_i)``
the singular triplets of the Newton-Schulz input N ("Muon is Scalable for
LLM Training", section 2.1, Eq. 2: the odd quintic acts on singular values
only, so the exact output has exactly ``f^N(sigma_i / ||N||)`` on its i-th
singular direction and nothing across directions).  The pins below fix it
to things other than itself:

* it is ~0 on the oracle's own iterated output;
* a planted perturbation ``delta u_k v_k^T`` reads back as exactly |delta|
  (max, not mean; a second, smaller plant does not change it);
* transposing both arguments leaves it unchanged;
* for a rectangular-diagonal N the singular triplets are coordinate axes, so
  the metric is ``max_i |X_ii - f^N(s_i / ||s||)|`` with the quintic
  iterated in 50-digit decimal arithmetic -- no SVD involved;
* planted mistakes (target not normalised, U and V swapped, mean instead of
  max, signed instead of absolute, wrong iteration count) each fail a pin.

``per_sigma_deviation_gram`` and ``ns_closed_form_gram`` take the same
triplets from the eigenproblem of the short-side Gram matrix (the route the
8192-class parity tests use); they are pinned to the SVD forms and to the
iterative oracle.
"""

from __future__ import annotations

import math
from decimal import Decimal, localcontext

import numpy as np
import pytest

from oracle import muon_oracle as mo, spectral as sp

ABC = mo.NS_COEFFS


def _rng(seed):
    return np.random.default_rng(seed)


def _dec_map(x: float, steps: int) -> float:
    with localcontext() as ctx:
        ctx.prec = 50
        a, b, c = (Decimal(str(v)) for v in ABC)
        y = Decimal(x)
        for _ in range(steps):
            y2 = y * y
            y = a * y + b * y2 * y + c * y2 * y2 * y
        return float(y)


def _ill(m, n, seed, lo=-6):
    r = _rng(seed)
    U, _ = np.linalg.qr(r.standard_normal((m, min(m, n))))
    V, _ = np.linalg.qr(r.standard_normal((n, min(m, n))))
    return (U * np.logspace(lo, 0, min(m, n))) @ V.T


SHAPES = [(24, 60), (60, 24), (40, 40), (1, 17), (17, 1)]


def _input(shape, seed):
    return _rng(seed).standard_normal(shape)


# ---------------------------------------------------------------- the SVD form

@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("steps", [1, 5, 10])
def test_zero_on_oracle_output(shape, steps):
    N = _input(shape, 3 * shape[0] + shape[1])
    X, _ = mo.orthogonalize(N, steps)
    assert sp.per_sigma_deviation(X, N, steps) <= 1e-12


@pytest.mark.parametrize("shape", [(24, 60), (60, 24), (40, 40)])
def test_planted_direction_reads_back(shape):
    N = _input(shape, 100 + shape[0])
    X, _ = mo.orthogonalize(N, 5)
    U, s, Vt = np.linalg.svd(N, full_matrices=False)
    m = s.size
    for k, delta in ((0, 0.037), (m // 2, -0.021), (m - 1, 0.0905)):
        Y = X + delta * np.outer(U[:, k], Vt[k])
        assert abs(sp.per_sigma_deviation(Y, N, 5) - abs(delta)) <= 1e-12
        # a second, smaller plant elsewhere: still the max
        j = (k + 1) % m
        Z = Y + 0.5 * delta * np.outer(U[:, j], Vt[j])
        assert abs(sp.per_sigma_deviation(Z, N, 5) - abs(delta)) <= 1e-12


@pytest.mark.parametrize("shape", [(24, 60), (40, 40)])
def test_transpose_invariant(shape):
    N = _input(shape, 200 + shape[0])
    X, _ = mo.orthogonalize(N, 5)
    Y = X + 0.01 * _rng(5).standard_normal(shape)
    a = sp.per_sigma_deviation(Y, N, 5)
    b = sp.per_sigma_deviation(Y.T, N.T, 5)
    assert a > 1e-3
    assert abs(a - b) <= 1e-12


def _diag_case():
    """N = rectangular diag(3, 2, 1) [3, 5]: u_i = e_i, v_i = e_i."""
    s = np.array([3.0, 2.0, 1.0])
    N = np.zeros((3, 5))
    N[0, 0], N[1, 1], N[2, 2] = s
    X = _rng(9).uniform(-1, 1, (3, 5))
    with localcontext() as ctx:
        ctx.prec = 50
        nu = Decimal(14).sqrt()
        targets = [_dec_map(Decimal(float(v)) / nu, 5) for v in s]
    expect = max(abs(X[i, i] - targets[i]) for i in range(3))
    return X, N, expect


def test_rectangular_diagonal_by_hand():
    X, N, expect = _diag_case()
    assert abs(sp.per_sigma_deviation(X, N, 5, eps=0.0) - expect) <= 1e-12
    assert abs(sp.per_sigma_deviation(X.T, N.T, 5, eps=0.0) - expect) <= 1e-12


# ---------------------------------------------------------------- mutants

def _pins_fail(fn) -> bool:
    """True when a planted-mistake version of the metric fails a pin."""
    try:
        for shape in [(24, 60), (40, 40)]:
            N = _input(shape, 300 + shape[0])
            X, _ = mo.orthogonalize(N, 5, eps=0.0)
            if fn(X, N, 5) > 1e-9:
                return True
            U, s, Vt = np.linalg.svd(N, full_matrices=False)
            Y = X + 0.037 * np.outer(U[:, 1], Vt[1])
            if abs(fn(Y, N, 5) - 0.037) > 1e-9:
                return True
        X, N, expect = _diag_case()
        if abs(fn(X, N, 5) - expect) > 1e-9:
            return True
    except Exception:
        return True
    return False


def _mut(kind):
    def f(X, N, steps, abc=ABC, eps=0.0):
        X = np.asarray(X, float)
        U, s, Vt = np.linalg.svd(N, full_matrices=False)
        nu = math.sqrt(float(np.sum(s * s))) + eps
        x = s if kind == "unnormalised" else s / nu
        target = sp.scalar_map(x, steps + (1 if kind == "steps" else 0), abc)
        if kind == "swap":
            proj = np.einsum("ij,ij->j", Vt.T[: N.shape[0]], X @ U[: N.shape[1]])
        else:
            proj = np.einsum("ij,ij->j", U, X @ Vt.T)
        d = proj - target
        if kind == "mean":
            return float(np.mean(np.abs(d)))
        if kind == "signed":
            return float(np.max(d))
        return float(np.max(np.abs(d)))
    return f


def test_metric_itself_passes_pins():
    assert not _pins_fail(lambda X, N, steps: sp.per_sigma_deviation(X, N, steps, eps=0.0))
    assert not _pins_fail(lambda X, N, steps: sp.per_sigma_deviation_gram(X, N, steps, eps=0.0))


@pytest.mark.filterwarnings("ignore:overflow encountered")   # the unnormalised mutant blows up
@pytest.mark.parametrize("kind", ["unnormalised", "swap", "mean", "signed", "steps"])
def test_metric_mutants_are_caught(kind):
    assert _pins_fail(_mut(kind)), kind


# ---------------------------------------------------------------- the Gram-eigen route

@pytest.mark.parametrize("shape", SHAPES + [(33, 200), (200, 33)])
@pytest.mark.parametrize("steps", [5, 10])
def test_gram_route_matches_svd_route(shape, steps):
    N = _input(shape, 400 + 5 * shape[0] + shape[1])
    X, _ = mo.orthogonalize(N, steps)
    Y = X + 0.02 * _rng(11).standard_normal(shape)
    a = sp.per_sigma_deviation(Y, N, steps)
    b = sp.per_sigma_deviation_gram(Y, N, steps)
    assert abs(a - b) <= 1e-10
    assert sp.per_sigma_deviation_gram(X, N, steps) <= 1e-10
    assert sp.rel_fro(sp.ns_closed_form_gram(N, steps), X) <= 1e-10


@pytest.mark.parametrize("shape", [(64, 160), (160, 64), (80, 80)])
@pytest.mark.parametrize("steps", [5, 10])
def test_gram_route_ill_conditioned(shape, steps):
    """Singular values spread over 1e-6 .. 1 (condition 1e6, beyond any
    Gaussian input here): the Gram matrix squares it, so eigenvalues near
    the bottom carry ~1e-16 * 1e12 relative error.  Measured: closed form
    1e-12 (N = 5) and 8e-8 (N = 10), metric 7e-9 and 3.3e-6; the bounds
    below sit four orders of magnitude under the 5e-2 parity gate."""
    N = _ill(*shape, seed=shape[0] + shape[1])
    X, _ = mo.orthogonalize(N, steps)
    assert sp.rel_fro(sp.ns_closed_form_gram(N, steps), X) <= (1e-10 if steps == 5 else 1e-6)
    assert sp.per_sigma_deviation_gram(X, N, steps) <= (1e-7 if steps == 5 else 1e-5)


def test_gram_route_zero_and_rank_deficient():
    N = np.zeros((8, 20))
    assert sp.per_sigma_deviation_gram(np.zeros((8, 20)), N, 5) == 0.0
    assert np.count_nonzero(sp.ns_closed_form_gram(N, 5)) == 0
    r = _rng(13)
    N = np.outer(r.standard_normal(12), r.standard_normal(30)) + \
        np.outer(r.standard_normal(12), r.standard_normal(30))       # rank 2
    X, _ = mo.orthogonalize(N, 5)
    assert sp.rel_fro(sp.ns_closed_form_gram(N, 5), X) <= 1e-10
    # rank-2 input: the Gram matrix returns its exact zeros as eigenvalues of
    # about 2^-52 sigma_1^2, i.e. singular values near 1e-8 sigma_1; a floor
    # of 1e-6 leaves those undefined directions out
    assert sp.per_sigma_deviation_gram(X, N, 5, rel_floor=1e-6) <= 1e-10


def test_gram_route_rel_floor_only_drops_small_directions():
    N = _ill(40, 90, seed=7, lo=-8)
    X, _ = mo.orthogonalize(N, 5)
    sigma, Q, _ = sp.short_side_eig(N)
    # plant on the smallest direction: visible without a floor, hidden with one
    u = Q[:, -1]
    v = N.T @ u / sigma[-1]
    v /= np.linalg.norm(v)
    Y = X + 0.05 * np.outer(u, v)
    assert sp.per_sigma_deviation_gram(Y, N, 5) >= 0.04
    assert sp.per_sigma_deviation_gram(Y, N, 5, rel_floor=1e-4) <= 1e-9
