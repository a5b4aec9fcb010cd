"""Plain fp64 CPU oracle of the Muon optimizer step and of the AdamW side path.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
link this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library (no kernels, headers, helpers or constants are common to both).

Every function works on numpy float64 arrays and follows the pages' steps in
their order, with numpy matmul as the only library primitive.

Sources ("Muon is Scalable for LLM Training", Moonshot AI / UCLA, 2025 --
the Traditional-Chinese translation page of the technical report):

* section 2.1, Eq. 1 -- momentum accumulation ``M_t = mu M_{t-1} + G_t`` with
  ``M_0 = 0`` and the parameter step through the Newton-Schulz output;
* section 2.1, paragraph after Eq. 1 -- the Nesterov-style variant feeds
  ``mu M_t + G_t`` (with the freshly updated ``M_t``) to Newton-Schulz;
* section 2.1, Eq. 2 and the text around it -- ``X_0 = M / ||M||_F`` and the
  quintic iteration ``X_k = a X + b (X X^T) X + c (X X^T)^2 X`` with
  ``(a, b, c) = (3.4445, -4.7750, 2.0315)``;
* section 2.2, Eq. 3 / Eq. 4 (= section 3.1, Eq. 7) -- decoupled weight decay
  and the shape scale ``0.2 * sqrt(max(A, B))``;
* section 2.2, "other hyper-parameters" -- N = 5 and mu = 0.95;
* section 2.3, Algorithm 1 -- the step reports ``sqrt(mean(u^2))`` of the
  update for logging;
* section 3.1, Eq. 5 and Eq. 6 -- the alternative update scalings
  ``0.2 * sqrt(H)`` (H the model's hidden size) and ``0.2 / RMS(O_t)``;
* section 2.2 (matching AdamW's update RMS) -- RMSNorm, embedding and LM head
  parameters use AdamW with the same learning rate and weight decay.

Readings where the pages leave a step open (each is also listed in the
design notes of the repository):

* epsilon: ``X_0 = M / (||M||_F + eps)`` so that a zero matrix yields a zero
  update (the pages divide by the norm exactly);
* orientation: for a tall matrix (rows > cols) the iteration runs on the
  transpose and the result is transposed back.  Because the iteration is an
  odd matrix polynomial this is exact in real arithmetic; it keeps the Gram
  matrix on the short side;
* the reported RMS is that of the unscaled Newton-Schulz output ``X_N``;
* Eq. 6 with ``O_t = 0`` (zero gradient history): ``O_t / RMS(O_t)`` is
  taken as zero, so the step is decay only (the same as the other scalings);
* AdamW's beta1, beta2, eps and bias correction are not printed on the pages
  (they only say "standard AdamW"): the defaults of the cited Adam paper
  (0.9, 0.999, 1e-8, with bias correction) are used, and the decay is applied
  to every AdamW tensor, RMSNorm gains included.
"""

from __future__ import annotations

import math

import numpy as np

# Section 2.1, coefficients given right after Eq. 2.
NS_COEFFS = (3.4445, -4.7750, 2.0315)
# Section 2.2, "other hyper-parameters": N = 5, momentum 0.95.
NS_STEPS = 5
MOMENTUM = 0.95
# Section 2.2, Eq. 4: target update RMS 0.2 via 0.2 * sqrt(max(A, B)).
RMS_SCALE = 0.2
# Normalisation guard (reading of Eq. 2's X_0 = M / ||M||_F for M = 0).
NORM_EPS = 1e-7


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def momentum_update(M, G, mu: float = MOMENTUM, nesterov: bool = True):
    """Momentum buffer update and Newton-Schulz input.

    Section 2.1, Eq. 1: ``M_t = mu * M_{t-1} + G_t``.  The Nesterov-style
    variant (the paragraph after Eq. 1) feeds ``mu * M_t + G_t`` -- built
    from the *updated* buffer -- to Newton-Schulz instead of ``M_t``.

    Returns ``(M_new, ns_input)``.
    """
    M = _f64(M)
    G = _f64(G)
    M_new = mu * M + G
    ns_input = mu * M_new + G if nesterov else M_new
    return M_new, ns_input


def frobenius_normalize(N, eps: float = NORM_EPS):
    """Section 2.1, text before Eq. 2: ``X_0 = N / ||N||_F`` (plus eps).

    Returns ``(X_0, nu)`` with ``nu = ||N||_F``.
    """
    N = _f64(N)
    nu = math.sqrt(float(np.sum(N * N)))
    return N / (nu + eps), nu


def newton_schulz(X0, steps: int = NS_STEPS, abc=NS_COEFFS):
    """Section 2.1, Eq. 2, iterated ``steps`` times from ``X0``.

    Each iteration forms the Gram matrix ``S = X X^T``, the polynomial
    ``P = b S + c S S`` (so that ``b (XX^T) X + c (XX^T)^2 X = P X``) and
    ``X <- a X + P X``.  A tall input is processed as its transpose (the
    Gram matrix is then the small ``min x min`` one) and transposed back.
    """
    a, b, c = (float(v) for v in abc)
    X = _f64(X0)
    tall = X.shape[0] > X.shape[1]
    if tall:
        X = X.T
    for _ in range(int(steps)):
        S = X @ X.T
        P = b * S + c * (S @ S)
        X = a * X + P @ X
    return X.T if tall else X


def orthogonalize(N, steps: int = NS_STEPS, abc=NS_COEFFS, eps: float = NORM_EPS):
    """Normalise then iterate: the ``Newton-Schulz(.)`` of section 2.1, Eq. 1.

    Returns ``(X_N, nu)``.
    """
    X0, nu = frobenius_normalize(N, eps)
    return newton_schulz(X0, steps, abc), nu


def shape_scale(rows: int, cols: int, rms_scale: float = RMS_SCALE) -> float:
    """Section 2.2, Eq. 4: the factor ``0.2 * sqrt(max(A, B))``."""
    return rms_scale * math.sqrt(max(rows, cols))


def apply_update(W, X_N, lr: float, wd: float, rms_scale: float = RMS_SCALE,
                 scaling: str = "shape", hidden=None):
    """The scaled, decoupled-decay update of one matrix.

    scaling "shape": section 2.2, Eq. 4 (= section 3.1, Eq. 7),
        ``W_t = W_{t-1} - lr * (0.2 * X_N * sqrt(max(A, B)) + wd * W_{t-1})``;
    scaling "hidden": section 3.1, Eq. 5, ``0.2 * X_N * sqrt(H)`` in place of
        the shape factor (``hidden`` = H);
    scaling "update_norm": section 3.1, Eq. 6, ``0.2 * X_N / RMS(X_N)``.
    The decay term uses the weights from before this step.
    """
    W = _f64(W)
    X_N = _f64(X_N)
    rows, cols = W.shape
    if scaling == "shape":
        U = shape_scale(rows, cols, rms_scale) * X_N
    elif scaling == "hidden":
        if hidden is None:
            raise ValueError("scaling 'hidden' needs H")
        U = rms_scale * math.sqrt(hidden) * X_N
    elif scaling == "update_norm":
        r = update_rms(X_N)
        U = rms_scale * X_N / r if r > 0.0 else np.zeros_like(X_N)
    else:
        raise ValueError(f"unknown scaling {scaling!r}")
    return W - lr * (U + wd * W)


def update_rms(X_N) -> float:
    """Section 2.3, Algorithm 1, its return value ``sqrt(mean(u^2))``
    (taken here over the unscaled Newton-Schulz output)."""
    X_N = _f64(X_N)
    return math.sqrt(float(np.mean(X_N * X_N)))


def muon_step(W, G, M, *, lr: float, wd: float, mu: float = MOMENTUM,
              nesterov: bool = True, ns_steps: int = NS_STEPS, abc=NS_COEFFS,
              rms_scale: float = RMS_SCALE, eps: float = NORM_EPS,
              scaling: str = "shape", hidden=None):
    """One Muon step for one matrix parameter ``W [A, B]``.

    Momentum (Eq. 1 + Nesterov), Frobenius normalisation and Newton-Schulz
    (Eq. 2), then the scaled, decoupled-decay update (Eq. 4; Eq. 5 or Eq. 6
    with ``scaling``).

    Returns ``(W_new, M_new, X_N, rms_of_X_N)``.
    """
    M_new, N = momentum_update(M, G, mu, nesterov)
    X_N, _ = orthogonalize(N, ns_steps, abc, eps)
    W_new = apply_update(W, X_N, lr, wd, rms_scale, scaling, hidden)
    return W_new, M_new, X_N, update_rms(X_N)


# AdamW defaults: the pages only say "standard AdamW"; these are the cited
# Adam paper's defaults (a reading, not a printed value).
ADAM_BETA1 = 0.9
ADAM_BETA2 = 0.999
ADAM_EPS = 1e-8


def adamw_step(W, g, m, v, *, lr: float, wd: float, beta1: float = ADAM_BETA1,
               beta2: float = ADAM_BETA2, eps: float = ADAM_EPS, t: int = 1):
    """AdamW for non-matrix parameters (section 2.2, matching AdamW's update
    RMS: RMSNorm, embedding and LM head stay on AdamW with the same lr and wd).

    Decoupled decay in the same form as Eq. 3 (``- lr * wd * W_{t-1}``),
    moments with bias correction at step ``t >= 1``.

    Returns ``(W_new, m_new, v_new)``.
    """
    if t < 1:
        raise ValueError("AdamW step counter starts at 1")
    W = _f64(W)
    g = _f64(g)
    m_new = beta1 * _f64(m) + (1.0 - beta1) * g
    v_new = beta2 * _f64(v) + (1.0 - beta2) * g * g
    m_hat = m_new / (1.0 - beta1 ** t)
    v_hat = v_new / (1.0 - beta2 ** t)
    W_new = W - lr * (m_hat / (np.sqrt(v_hat) + eps) + wd * W)
    return W_new, m_new, v_new

