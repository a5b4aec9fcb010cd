"""Pure-Python brute force of one Muon step, for tiny matrices.

TEST INFRASTRUCTURE ONLY (see ``muon_oracle``'s header).

No numpy: nested lists of Python floats and explicit triple loops.  It
evaluates Eq. 2 of "Muon is Scalable for LLM Training" (section 2.1) term by
term, ``a X + b (X X^T) X + c (X X^T)(X X^T) X``, on the matrix as given --
without the short-side orientation and without the grouping into
``P = b S + c S^2`` that the numpy oracle uses -- so that it checks those
choices as well as the arithmetic.
"""

from __future__ import annotations

import math


def _matmul(A, B):
    n, k, m = len(A), len(B), len(B[0])
    out = []
    for i in range(n):
        row = []
        for j in range(m):
            acc = 0.0
            for t in range(k):
                acc += A[i][t] * B[t][j]
            row.append(acc)
        out.append(row)
    return out


def _transpose(A):
    return [list(col) for col in zip(*A)]


def _axpby(alpha, A, beta, B):
    return [[alpha * x + beta * y for x, y in zip(ra, rb)] for ra, rb in zip(A, B)]


def _scale(alpha, A):
    return [[alpha * x for x in r] for r in A]


def ns_literal(X0, steps, abc):
    """Eq. 2 with every term formed separately."""
    a, b, c = abc
    X = [list(map(float, r)) for r in X0]
    for _ in range(steps):
        G = _matmul(X, _transpose(X))          # X X^T
        GX = _matmul(G, X)                      # (X X^T) X
        GGX = _matmul(G, GX)                    # (X X^T)^2 X
        X = [[a * x + b * gx + c * ggx for x, gx, ggx in zip(rx, rgx, rggx)]
             for rx, rgx, rggx in zip(X, GX, GGX)]
    return X


def muon_step(W, G, M, *, lr, wd, mu, nesterov, ns_steps, abc, rms_scale, eps):
    """Eq. 1 (+ Nesterov), Eq. 2, Eq. 4, element by element.

    Returns ``(W_new, M_new, X_N, rms)`` as nested lists / a float.
    """
    rows, cols = len(W), len(W[0])
    M_new = _axpby(mu, M, 1.0, G)
    N = _axpby(mu, M_new, 1.0, G) if nesterov else [r[:] for r in M_new]
    sq = 0.0
    for r in N:
        for x in r:
            sq += x * x
    X0 = _scale(1.0 / (math.sqrt(sq) + eps), N)
    X = ns_literal(X0, ns_steps, abc)
    scale = rms_scale * math.sqrt(max(rows, cols))
    W_new = [[w - lr * (scale * x + wd * w) for w, x in zip(rw, rx)]
             for rw, rx in zip(W, X)]
    ss = 0.0
    for r in X:
        for x in r:
            ss += x * x
    return W_new, M_new, X, math.sqrt(ss / (rows * cols))


def adamw_step(W, g, m, v, *, lr, wd, beta1, beta2, eps, t):
    """Per-element AdamW with bias correction and decoupled decay."""
    W_new, m_new, v_new = [], [], []
    c1 = 1.0 - beta1 ** t
    c2 = 1.0 - beta2 ** t
    for w, gg, mm, vv in zip(W, g, m, v):
        mm = beta1 * mm + (1.0 - beta1) * gg
        vv = beta2 * vv + (1.0 - beta2) * gg * gg
        upd = (mm / c1) / (math.sqrt(vv / c2) + eps)
        W_new.append(w - lr * (upd + wd * w))
        m_new.append(mm)
        v_new.append(vv)
    return W_new, m_new, v_new
