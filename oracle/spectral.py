"""Spectral (SVD) closed form of the Newton-Schulz step and the per-singular-
value parity metric.

TEST INFRASTRUCTURE ONLY (see ``muon_oracle``'s header): used by ``tests/``
and ``bench.py``'s parity sampling, never by the product path.

Why a closed form exists ("Muon is Scalable for LLM Training", section 2.1,
Eq. 1 and Eq. 2): with ``X_0 = U S V^T`` (thin SVD), ``X X^T = U S^2 U^T``,
so one iteration maps ``U S V^T`` to ``U (a S + b S^3 + c S^5) V^T``.  The
singular vectors never move; every singular value goes through the scalar
quintic ``f(x) = a x + b x^3 + c x^5`` (the polynomial the pages name when
they discuss the coefficients), ``N`` times.  This route uses LAPACK's SVD
instead of any matrix product of the iteration, so it pins the iterative
oracle independently.  The same section says Newton-Schulz approximates
``U V^T``; ``polar_factor`` returns that exact target for Lemma-1 checks.
"""

from __future__ import annotations

import numpy as np

from .muon_oracle import NORM_EPS, NS_COEFFS, NS_STEPS


def scalar_map(x, steps: int = NS_STEPS, abc=NS_COEFFS):
    """Iterate ``f(x) = a x + b x^3 + c x^5`` (section 2.1) ``steps`` times."""
    a, b, c = (float(v) for v in abc)
    y = np.asarray(x, dtype=np.float64).copy()
    for _ in range(int(steps)):
        y2 = y * y
        y = y * (a + y2 * (b + c * y2))
    return y


def ns_closed_form(N, steps: int = NS_STEPS, abc=NS_COEFFS, eps: float = NORM_EPS):
    """``Newton-Schulz(N / (||N||_F + eps))`` via ``U f^N(S) V^T``."""
    N = np.asarray(N, dtype=np.float64)
    U, s, Vt = np.linalg.svd(N, full_matrices=False)
    nu = float(np.sqrt(np.sum(s * s)))
    y = scalar_map(s / (nu + eps), steps, abc)
    return (U * y) @ Vt


def polar_factor(N):
    """``U V^T`` of the thin SVD (the exact target of section 2.1)."""
    U, _, Vt = np.linalg.svd(np.asarray(N, dtype=np.float64), full_matrices=False)
    return U @ Vt


def per_sigma_deviation(X, N, steps: int = NS_STEPS, abc=NS_COEFFS,
                        eps: float = NORM_EPS) -> float:
    """``max_i |u_i^T X v_i - f^N(sigma_i / (||N|| + eps))|``.

    ``u_i, v_i, sigma_i`` come from the fp64 SVD of the Newton-Schulz input
    ``N``; ``X`` is a computed Newton-Schulz output of the same shape.  This
    measures how far each singular direction of ``X`` is from its exact
    polynomial image.
    """
    N = np.asarray(N, dtype=np.float64)
    X = np.asarray(X, dtype=np.float64)
    U, s, Vt = np.linalg.svd(N, full_matrices=False)
    nu = float(np.sqrt(np.sum(s * s)))
    target = scalar_map(s / (nu + eps), steps, abc)
    proj = np.einsum("ij,ij->j", U, X @ Vt.T)
    return float(np.max(np.abs(proj - target))) if s.size else 0.0


def rel_fro(x, ref) -> float:
    """Relative Frobenius error ``||x - ref||_F / ||ref||_F`` (0/0 -> 0)."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = float(np.linalg.norm(ref))
    num = float(np.linalg.norm(x - ref))
    if den == 0.0:
        return num
    return num / den
