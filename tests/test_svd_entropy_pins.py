"""Pins of the SVD-entropy oracle against things other than itself.

Section 3.4 of "Muon is Scalable for LLM Training" defines the SVD entropy of
a weight matrix from its squared singular values; appendix F plots the
singular values sorted from largest to smallest, divided by the largest.
The pins tie ``oracle.svd_entropy`` to:

* 2 x 2 matrices whose squared singular values are the roots of
  ``t^2 - ||M||_F^2 t + det(M)^2`` (no SVD routine involved), so that the
  entropy is a binary entropy with a known value (h(0.2), h(0.1) in bits);
* spectra fixed by construction: orthonormal rows (flat: H = 1), rank one
  (H = 0), r equal singular values (H = log r / log n), and signed,
  permuted Sylvester-Hadamard products ``H_m diag(s) P`` whose singular
  values are exactly ``sqrt(m) |s|``;
* invariances of singular values (transpose, orthogonal factors, scale);
* the readings for n = 1 and for the zero matrix.

``test_entropy_mutants_are_caught`` plants typical mistakes in copies of the
oracle and checks that at least one pin fails for each.
"""

from __future__ import annotations

import math

import numpy as np

from oracle import svd_entropy as se

# Binary entropies in bits (the n = 2 normaliser is log 2): h(0.2) and h(0.1).
H_BIN_02 = 0.72192809488736234787
H_BIN_01 = 0.46899559358928122125
# -(16/25 ln 16/25 + 9/25 ln 9/25) / ln 3, evaluated to 50 digits.
H_3_4_0 = 0.59476687229292329542


def hadamard(m: int) -> np.ndarray:
    """Sylvester's Hadamard matrix of order m (a power of two): H H^T = m I."""
    h = np.ones((1, 1))
    while h.shape[0] < m:
        h = np.block([[h, h], [h, -h]])
    return h


def hadamard_matrix(m: int, n: int, s: np.ndarray, rng) -> np.ndarray:
    """[m, n] (n >= m) matrix with singular values sqrt(m) |s|: H_m diag(s)
    placed on m of the n columns, then a random signed column permutation."""
    w = np.zeros((m, n))
    w[:, :m] = hadamard(m) * s[None, :]
    perm = rng.permutation(n)
    signs = rng.choice([-1.0, 1.0], size=n)
    return w[:, perm] * signs[None, :]


def orthonormal_rows(m: int, n: int, rng) -> np.ndarray:
    q, _ = np.linalg.qr(rng.standard_normal((n, m)))
    return q.T


def _pins(entropy, spectrum):
    """Runs every pin with the given functions; yields (name, ok)."""
    rng = np.random.default_rng(7)
    yield "diag(2,1)", abs(entropy(np.diag([2.0, 1.0])) - H_BIN_02) < 1e-14
    # [[3,0],[4,5]]: ||M||_F^2 = 50, det = 15 -> t in {45, 5}: p = (0.9, 0.1)
    yield "2x2 char poly", abs(entropy(np.array([[3.0, 0.0], [4.0, 5.0]])) - H_BIN_01) < 1e-14
    yield "diag(3,-4,0)", abs(entropy(np.diag([3.0, -4.0, 0.0])) - H_3_4_0) < 1e-14
    sp = spectrum(np.diag([3.0, -4.0, 0.0]))
    yield "curve diag(3,-4,0)", sp.shape == (3,) and np.allclose(sp, [1.0, 0.75, 0.0], rtol=0, atol=1e-15)
    for m, n in ((4, 8), (5, 5), (16, 40)):
        q = 3.0 * orthonormal_rows(m, n, rng)
        yield f"flat {m}x{n}", abs(entropy(q) - 1.0) < 1e-12
        yield f"flat {n}x{m}", abs(entropy(q.T) - 1.0) < 1e-12
        yield f"flat curve {m}x{n}", np.allclose(spectrum(q), np.ones(m), rtol=0, atol=1e-12)
    u, v = rng.standard_normal(6), rng.standard_normal(9)
    yield "rank one", abs(entropy(np.outer(u, v))) < 1e-12
    for r, m, n in ((2, 6, 10), (3, 8, 8), (5, 7, 12)):
        # [m, r] orthonormal columns times [r, n] orthonormal rows: r unit
        # singular values, the other m - r zero
        flat_r = orthonormal_rows(r, m, rng).T @ orthonormal_rows(r, n, rng)
        yield f"rank {r} flat {m}x{n}", abs(entropy(flat_r) - math.log(r) / math.log(m)) < 1e-12
    for m, n in ((8, 8), (16, 48), (32, 33)):
        s = rng.uniform(-2.0, 2.0, size=m)
        w = hadamard_matrix(m, n, s, rng)
        sq = s * s
        p = sq / sq.sum()
        want = -float(np.sum(p * np.log(p))) / math.log(m)
        yield f"hadamard {m}x{n}", abs(entropy(w) - want) < 1e-12 and abs(entropy(w.T) - want) < 1e-12
        want_curve = np.sort(np.abs(s))[::-1] / np.max(np.abs(s))
        yield f"hadamard curve {m}x{n}", np.allclose(spectrum(w), want_curve, rtol=0, atol=1e-12)
    w = rng.standard_normal((7, 11))
    qa = orthonormal_rows(7, 7, rng)
    qb = orthonormal_rows(11, 11, rng)
    h0 = entropy(w)
    yield "invariance", (abs(entropy(w.T) - h0) < 1e-12 and abs(entropy(-3.5 * w) - h0) < 1e-12
                         and abs(entropy(qa @ w @ qb) - h0) < 1e-12 and 0.0 < h0 < 1.0)
    yield "n = 1", entropy(np.arange(1.0, 6.0)[None, :]) == 0.0 and entropy(np.ones((4, 1))) == 0.0
    yield "zero matrix", entropy(np.zeros((3, 5))) == 0.0 and np.all(spectrum(np.zeros((3, 5))) == 0.0)


def _failures(entropy, spectrum):
    return [name for name, ok in _pins(entropy, spectrum) if not ok]


def test_oracle_pins():
    assert _failures(se.svd_entropy, se.normalized_spectrum) == []


def test_singular_values_descending_and_count():
    rng = np.random.default_rng(3)
    for shape in ((5, 9), (9, 5), (6, 6), (1, 4)):
        s = se.singular_values(rng.standard_normal(shape))
        assert s.shape == (min(shape),)
        assert np.all(np.diff(s) <= 0)


def test_entropy_mutants_are_caught():
    def unsquared(w):                        # p from sigma, not sigma^2
        s = se.singular_values(w)
        return se.entropy_from_sigma(np.sqrt(s))

    def log_max(w):                          # normaliser log max(A, B)
        h = se.svd_entropy(w)
        n, big = min(np.shape(w)), max(np.shape(w))
        return h * math.log(n) / math.log(big) if n > 1 else h

    def no_normaliser(w):
        n = min(np.shape(w))
        return se.svd_entropy(w) * (math.log(n) if n > 1 else 1.0)

    def row_norms(w):                        # row norms instead of singular values
        w = np.asarray(w, dtype=np.float64)
        w = w if w.shape[0] <= w.shape[1] else w.T
        return se.entropy_from_sigma(np.linalg.norm(w, axis=1))

    def ascending(w):                        # curve sorted the wrong way
        return se.normalized_spectrum(w)[::-1]

    def by_last(w):                          # curve divided by the smallest
        s = se.singular_values(w)
        return s / s[-1] if s[-1] != 0 else s

    for ent in (unsquared, log_max, no_normaliser, row_norms):
        assert _failures(ent, se.normalized_spectrum), ent.__name__
    for spec in (ascending, by_last):
        assert _failures(se.svd_entropy, spec), spec.__name__
