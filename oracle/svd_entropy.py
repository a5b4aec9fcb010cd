"""SVD entropy and normalised singular-value curve of a matrix (fp64).

TEST INFRASTRUCTURE ONLY (see ``muon_oracle``'s header): used by ``tests/``,
``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg, never by
the product path.  It shares no code with the HIP library.

Source: "Muon is Scalable for LLM Training" (Moonshot AI / UCLA, 2025), the
Traditional-Chinese translation page of the technical report:

* section 3.4 (singular-value spectrum dynamics), the SVD-entropy equation:
  for singular values ``sigma_1 .. sigma_n`` of a weight matrix, with
  ``p_i = sigma_i^2 / sum_j sigma_j^2``, the entropy is
  ``H = -(1 / log n) * sum_i p_i log p_i`` -- the Shannon entropy of the
  squared-singular-value distribution, normalised so that a flat spectrum
  gives 1;
* appendix F (singular-value distribution of the weight matrices): the
  singular values are sorted from largest to smallest and divided by the
  largest one.

This is the plain definition written out: the singular values come from
LAPACK's SVD (numpy, fp64) and the sum is taken in the order given.

Readings where the pages leave a point open (also listed in the design
notes of the repository):

* ``n`` is the number of singular values of an ``[A, B]`` matrix,
  ``min(A, B)``; zero singular values count in ``n`` and contribute
  ``0 log 0 = 0`` (the limit);
* ``n = 1`` makes the normaliser ``log 1 = 0``: the entropy is taken as 0
  (one direction carries all of the spectrum);
* an all-zero matrix has no distribution: its entropy is taken as 0 and its
  normalised curve as all zeros.
"""

from __future__ import annotations

import math

import numpy as np


def singular_values(W) -> np.ndarray:
    """Singular values of ``W`` in decreasing order, fp64 (``min(A, B)`` of them)."""
    W = np.asarray(W, dtype=np.float64)
    if W.ndim != 2:
        raise ValueError("expected a matrix")
    return np.linalg.svd(W, compute_uv=False)


def entropy_from_sigma(sigma) -> float:
    """Section 3.4's SVD entropy of the singular values ``sigma``."""
    s = np.asarray(sigma, dtype=np.float64)
    n = s.size
    if n <= 1:
        return 0.0
    sq = s * s
    total = float(np.sum(sq))
    if total == 0.0:
        return 0.0
    h = 0.0
    for x in sq:
        p = float(x) / total
        if p > 0.0:
            h -= p * math.log(p)
    return h / math.log(n)


def svd_entropy(W) -> float:
    """Section 3.4: the SVD entropy of the matrix ``W``."""
    return entropy_from_sigma(singular_values(W))


def normalized_spectrum(W) -> np.ndarray:
    """Appendix F: singular values, largest first, divided by the largest."""
    s = singular_values(W)
    if s.size == 0 or s[0] == 0.0:
        return np.zeros_like(s)
    return s / s[0]
