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


def short_side_eig(N):
    """Singular values and short-side singular vectors of ``N`` from the
    symmetric eigenproblem of its short-side Gram matrix.

    For ``N [A, B]`` with ``A <= B``: ``N N^T = U diag(sigma^2) U^T``, so the
    eigenvectors are the left singular vectors; for ``A > B`` the Gram matrix
    is ``N^T N`` and they are the right singular vectors.  Eigenvalues that
    rounding pushed below zero are clipped.  Returns ``(sigma, Q, tall)``
    with ``sigma`` largest first and ``Q``'s columns the matching vectors.
    This is the same factorisation as the thin SVD (an identity, not an
    approximation) at the cost of one product and one eigensolve, which is
    what makes 8192-class matrices affordable in fp64.
    """
    N = np.asarray(N, dtype=np.float64)
    tall = N.shape[0] > N.shape[1]
    G = N.T @ N if tall else N @ N.T
    lam, Q = np.linalg.eigh(G)
    order = np.argsort(lam)[::-1]
    lam, Q = lam[order], Q[:, order]
    return np.sqrt(np.maximum(lam, 0.0)), Q, tall


def _map_over_x(y_over, x, steps, abc):
    """``f^N(x) / x`` elementwise, with its limit ``a^N`` at ``x = 0``."""
    a = float(abc[0])
    out = np.full_like(x, a ** int(steps))
    nz = x > 0.0
    out[nz] = y_over(x[nz]) / x[nz]
    return out


def ns_closed_form_gram(N, steps: int = NS_STEPS, abc=NS_COEFFS,
                        eps: float = NORM_EPS, eig=None):
    """The closed form of ``ns_closed_form`` taken through ``short_side_eig``.

    ``U f^N(S / nu) V^T = U diag(f^N(sigma_i / nu) / sigma_i) U^T N`` (wide;
    ``N Q diag(.) Q^T`` when tall), since ``V^T = S^{-1} U^T N``.  The ratio
    ``f^N(x) / x`` is smooth down to ``x = 0`` (limit ``a^N``), so directions
    with tiny or zero singular values need no special care.
    """
    N = np.asarray(N, dtype=np.float64)
    sigma, Q, tall = short_side_eig(N)
    nu = float(np.sqrt(np.sum(N * N)))
    x = sigma / (nu + eps)
    h = _map_over_x(lambda t: scalar_map(t, steps, abc), x, steps, abc) / (nu + eps)
    K = (Q * h) @ Q.T
    return N @ K if tall else K @ N


def per_sigma_projections_gram(X, N, eig=None):
    """``(sigma, u_i^T X v_i)`` for every singular triplet of ``N`` with
    ``sigma_i > 0`` (see ``per_sigma_deviation_gram``), largest first."""
    N = np.asarray(N, dtype=np.float64)
    X = np.asarray(X, dtype=np.float64)
    if N.shape != X.shape:
        raise ValueError("X and N must have the same shape")
    sigma, Q, tall = short_side_eig(N) if eig is None else eig
    keep = sigma > 0.0
    B = X.T @ N if tall else X @ N.T               # short x short
    Qk = Q[:, keep]
    return sigma[keep], np.einsum("ij,ij->j", Qk, B @ Qk) / sigma[keep]


def per_sigma_deviation_gram(X, N, steps: int = NS_STEPS, abc=NS_COEFFS,
                             eps: float = NORM_EPS, rel_floor: float = 0.0,
                             eig=None) -> float:
    """``per_sigma_deviation`` with the singular triplets of ``N`` from
    ``short_side_eig``.

    With ``u_i`` a short-side singular vector and ``sigma_i > 0``, the
    long-side partner is ``v_i = N^T u_i / sigma_i`` (wide), so
    ``u_i^T X v_i = u_i^T (X N^T) u_i / sigma_i`` and only one product with
    ``N`` is needed.  Directions with ``sigma_i <= rel_floor * sigma_1`` (and
    exact zeros, whose partner is undefined) are left out; the Gram matrix
    returns exact zeros of N as singular values near ``1e-8 sigma_1``, so a
    rank-deficient input needs a floor above that.  ``eig``:
    ``short_side_eig(N)`` if already computed.
    """
    N = np.asarray(N, dtype=np.float64)
    sig, proj = per_sigma_projections_gram(X, N, eig)
    nu = float(np.sqrt(np.sum(N * N)))
    keep = sig > rel_floor * (sig[0] if sig.size else 0.0)
    if not np.any(keep):
        return 0.0
    target = scalar_map(sig[keep] / (nu + eps), steps, abc)
    return float(np.max(np.abs(proj[keep] - target)))


def rel_fro(x, ref) -> float:
    """Relative Frobenius error ``||x - ref||_F / ||ref||_F`` (0/0 -> 0)."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = float(np.linalg.norm(ref))
    num = float(np.linalg.norm(x - ref))
    if den == 0.0:
        return num
    return num / den
