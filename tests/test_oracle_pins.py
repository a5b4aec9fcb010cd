"""Pins of the fp64 oracle against things other than itself.

Each test ties the oracle to something the pages or mathematics fix:

* the pages' printed constants (``tests/golden/pages_constants.json``);
* a pure-Python brute force that evaluates Eq. 2 term by term without the
  oracle's short-side orientation or its ``P = bS + cS^2`` grouping;
* the SVD closed form ``U f^N(S/||N||) V^T`` (Eq. 2 is an odd matrix
  polynomial, so it acts on singular values only);
* special inputs with exact answers computed in rational arithmetic
  (rank one, orthonormal rows, rectangular diagonal, zero);
* invariances (transpose, orthogonal factors, positive scale, sign);
* Lemma 1 (section 2.2 / appendix A) tying the shape scale to RMS 0.2;
* closed forms of the momentum recurrence (Eq. 1) and of AdamW under a
  constant gradient (bias correction makes every step identical).

``test_mutants_are_caught`` plants typical mistakes in copies of the
oracle's functions and checks that at least one pin fails for each.
"""

from __future__ import annotations

import json
import math
import os
from decimal import Decimal, localcontext

import numpy as np
import pytest

from oracle import brute, muon_oracle as mo, spectral as sp

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_constants.json")
ABC = mo.NS_COEFFS


def _rng(seed):
    return np.random.default_rng(seed)


def _dec_map(x, steps: int, abc=ABC) -> float:
    """The scalar quintic of section 2.1 iterated in 50-digit decimal
    arithmetic (the coefficients taken exactly as printed)."""
    with localcontext() as ctx:
        ctx.prec = 50
        a, b, c = (Decimal(str(v)) for v in abc)
        x = Decimal(x) if not isinstance(x, Decimal) else x
        for _ in range(steps):
            x2 = x * x
            x = a * x + b * x2 * x + c * x2 * x2 * x
        return float(x)


def _dec_inv_sqrt(m: int) -> Decimal:
    with localcontext() as ctx:
        ctx.prec = 50
        return Decimal(1) / Decimal(m).sqrt()


def _orthonormal_rows(m, n, seed):
    q, _ = np.linalg.qr(_rng(seed).standard_normal((n, m)))
    return q.T.copy()          # [m, n] with Q Q^T = I_m


# ---------------------------------------------------------------- constants

def test_constants_match_pages():
    g = json.load(open(GOLDEN))
    assert mo.NS_COEFFS == (g["ns_coefficients"]["a"], g["ns_coefficients"]["b"],
                            g["ns_coefficients"]["c"])
    assert mo.NS_STEPS == g["ns_steps"]["value"]
    assert mo.MOMENTUM == g["momentum"]["value"]
    assert mo.RMS_SCALE == g["update_rms_target"]["value"]


# ---------------------------------------------------------------- brute force

HYPER = dict(lr=1e-3, wd=0.1, mu=0.95, nesterov=True, ns_steps=5, abc=ABC,
             rms_scale=0.2, eps=1e-7)


@pytest.mark.parametrize("shape", [(4, 8), (8, 4), (3, 5), (5, 5), (1, 6), (6, 1), (2, 7)])
@pytest.mark.parametrize("variant", [{}, {"nesterov": False}, {"ns_steps": 0},
                                     {"ns_steps": 1}, {"ns_steps": 10}])
def test_brute_force_matches_oracle(shape, variant):
    r = _rng(hash((shape, tuple(variant.items()))) & 0xFFFF)
    W = r.normal(0, 0.02, shape)
    G = r.normal(0, 1.0, shape)
    M = r.normal(0, 0.5, shape)
    h = dict(HYPER, **variant)
    o = mo.muon_step(W, G, M, **h)
    b = brute.muon_step(W.tolist(), G.tolist(), M.tolist(), **h)
    for x, y in zip(o[:3], b[:3]):
        np.testing.assert_allclose(x, np.array(y), rtol=1e-11, atol=1e-14)
    assert abs(o[3] - b[3]) <= 1e-12 * max(1.0, abs(b[3]))


# ---------------------------------------------------------------- closed form

CF_SHAPES = [(64, 256), (256, 64), (128, 512), (96, 96), (200, 300), (300, 200), (1, 40)]


@pytest.mark.parametrize("shape", CF_SHAPES)
@pytest.mark.parametrize("steps", [1, 5, 10])
def test_closed_form_gaussian(shape, steps):
    N = _rng(shape[0] * 7 + shape[1]).standard_normal(shape)
    X, _ = mo.orthogonalize(N, steps)
    ref = sp.ns_closed_form(N, steps)
    assert sp.rel_fro(X, ref) < 1e-10


def test_closed_form_ill_conditioned():
    r = _rng(3)
    U, _ = np.linalg.qr(r.standard_normal((80, 80)))
    V, _ = np.linalg.qr(r.standard_normal((160, 80)))
    s = np.logspace(-6, 0, 80)
    N = (U * s) @ V.T
    for steps in (5, 10):
        X, _ = mo.orthogonalize(N, steps)
        assert sp.rel_fro(X, sp.ns_closed_form(N, steps)) < 1e-9


# ---------------------------------------------------------------- special inputs

@pytest.mark.parametrize("steps", [1, 5, 10])
def test_rank_one(steps):
    r = _rng(11)
    u, v = r.standard_normal(12), r.standard_normal(30)
    N = np.outer(u, v)
    X, _ = mo.orthogonalize(N, steps, eps=0.0)
    expect = _dec_map(1, steps)
    ref = expect * np.outer(u / np.linalg.norm(u), v / np.linalg.norm(v))
    # round-off in the null space (~1e-16) is lifted by about a^N per the
    # scalar map's slope at 0, so the bound grows with N
    assert sp.rel_fro(X, ref) < 1e-13 * ABC[0] ** steps
    # published-coefficient values of the scalar map at 1
    if steps == 5:
        assert abs(expect - 0.6964364095) < 1e-9


@pytest.mark.parametrize("m,n", [(4, 8), (16, 40), (64, 256)])
def test_orthonormal_rows(m, n):
    Q = _orthonormal_rows(m, n, m)
    x0 = _dec_inv_sqrt(m)                       # ||Q||_F = sqrt(m)
    for steps in (5, 10):
        X, _ = mo.orthogonalize(Q, steps, eps=0.0)
        ref = _dec_map(x0, steps) * Q
        assert sp.rel_fro(X, ref) < 1e-12
        Xt, _ = mo.orthogonalize(Q.T, steps, eps=0.0)
        assert sp.rel_fro(Xt, ref.T) < 1e-12


def test_rectangular_diagonal():
    d = np.array([3.0, 1.0, 0.25, 1e-3, 0.0])
    D = np.zeros((5, 9))
    D[np.arange(5), np.arange(5)] = d
    with localcontext() as ctx:
        ctx.prec = 50
        nu = sum(Decimal(float(x)) ** 2 for x in d).sqrt()
    X, _ = mo.orthogonalize(D, 5, eps=0.0)
    off = X.copy()
    off[np.arange(5), np.arange(5)] = 0.0
    assert np.all(off == 0.0)
    for i, di in enumerate(d):
        with localcontext() as ctx:
            ctx.prec = 50
            x0 = Decimal(float(di)) / nu
        ref = _dec_map(x0, 5)
        assert abs(X[i, i] - ref) <= 1e-12 * max(1.0, abs(ref))


def test_zero_matrix_gives_decay_only_step():
    W = _rng(5).normal(0, 0.02, (6, 10))
    Z = np.zeros_like(W)
    W1, M1, X, rms = mo.muon_step(W, Z, Z, **HYPER)
    assert np.all(X == 0.0) and np.all(M1 == 0.0) and rms == 0.0
    # decay invariant of Eq. 3/4: W - W' = lr * wd * W
    np.testing.assert_allclose(W1, W - HYPER["lr"] * HYPER["wd"] * W, rtol=4e-16, atol=0)


# ---------------------------------------------------------------- invariances

def test_invariances():
    r = _rng(17)
    N = r.standard_normal((24, 56))
    X, _ = mo.orthogonalize(N, 5)
    Xt, _ = mo.orthogonalize(N.T, 5)
    assert sp.rel_fro(Xt, X.T) < 1e-12
    Q1, _ = np.linalg.qr(r.standard_normal((24, 24)))
    Q2, _ = np.linalg.qr(r.standard_normal((56, 56)))
    Xq, _ = mo.orthogonalize(Q1 @ N @ Q2, 5)
    assert sp.rel_fro(Xq, Q1 @ X @ Q2) < 1e-10
    Xs, _ = mo.orthogonalize(37.5 * N, 5, eps=0.0)
    X0, _ = mo.orthogonalize(N, 5, eps=0.0)
    assert sp.rel_fro(Xs, X0) < 1e-12
    Xn, _ = mo.orthogonalize(-N, 5)
    assert sp.rel_fro(Xn, -X) < 1e-14


# ---------------------------------------------------------------- Lemma 1 / scale

@pytest.mark.parametrize("shape", [(64, 256), (256, 64), (100, 100), (30, 500)])
def test_lemma1_shape_scale_gives_rms_0p2(shape):
    """With the exact polar factor U V^T (the target of section 2.1), Eq. 4's
    update ``0.2 * sqrt(max(A,B)) * U V^T`` has RMS exactly 0.2 (Lemma 1)."""
    r = _rng(shape[0] + 3 * shape[1])
    W = r.normal(0, 0.02, shape)
    O = sp.polar_factor(r.standard_normal(shape))
    lr, wd = 1e-3, 0.1
    W1 = mo.apply_update(W, O, lr, wd)
    upd = (W - W1) / lr - wd * W
    assert abs(math.sqrt(np.mean(upd ** 2)) - 0.2) < 1e-10
    # Lemma 1 itself on the oracle's RMS: sqrt(r/(m n)) at full rank r=min
    assert abs(mo.update_rms(O) - 1.0 / math.sqrt(max(shape))) < 1e-12


def test_lemma1_rank_deficient_rms():
    r = _rng(23)
    m, n, k = 40, 90, 13
    U, _ = np.linalg.qr(r.standard_normal((m, k)))
    V, _ = np.linalg.qr(r.standard_normal((n, k)))
    X = U @ V.T
    assert abs(mo.update_rms(X) - math.sqrt(k / (m * n))) < 1e-13


@pytest.mark.parametrize("m,n", [(4, 8), (64, 256)])
def test_update_rms_of_full_step(m, n):
    """Orthonormal-row momentum input: the step's scaled update RMS is
    ``0.2 * f^N(1/sqrt(m))`` (Lemma 1 with r = m, times Eq. 4's scale)."""
    Q = _orthonormal_rows(m, n, 3)
    W = _rng(9).normal(0, 0.02, (m, n))
    G = Q / (1.0 + 0.95)                       # Nesterov input = (1+mu) G = Q
    h = dict(HYPER, eps=0.0)
    W1, _, X, rms = mo.muon_step(W, G, np.zeros_like(W), **h)
    upd = (W - W1) / h["lr"] - h["wd"] * W
    fx = _dec_map(_dec_inv_sqrt(m), 5)
    assert abs(math.sqrt(np.mean(upd ** 2)) - 0.2 * fx) < 1e-12
    assert abs(rms - fx / math.sqrt(n)) < 1e-13


# ---------------------------------------------------------------- Eq. 5 / Eq. 6 scalings

@pytest.mark.parametrize("shape", [(64, 256), (256, 64), (50, 50)])
def test_eq5_hidden_scale(shape):
    """Section 3.1, Eq. 5: with H = max(A, B) it is Eq. 4 exactly; with the
    exact polar factor (Lemma 1: RMS 1/sqrt(max(A, B))) the update RMS is
    0.2 sqrt(H / max(A, B)) for any H."""
    r = _rng(5 + shape[0] + shape[1])
    W = r.normal(0, 0.02, shape)
    O = sp.polar_factor(r.standard_normal(shape))
    lr, wd = 1e-3, 0.1
    a = mo.apply_update(W, O, lr, wd, scaling="hidden", hidden=max(shape))
    b = mo.apply_update(W, O, lr, wd)
    assert np.array_equal(a, b)
    for H in (128, 1536, 7):
        W1 = mo.apply_update(W, O, lr, wd, scaling="hidden", hidden=H)
        upd = (W - W1) / lr - wd * W
        assert abs(math.sqrt(np.mean(upd ** 2)) - 0.2 * math.sqrt(H / max(shape))) < 1e-10


@pytest.mark.parametrize("shape,rank", [((64, 256), 64), ((256, 64), 20), ((40, 40), 3), ((1, 300), 1)])
def test_eq6_update_norm_rms_is_0p2(shape, rank):
    """Section 3.1, Eq. 6: the update term 0.2 O / RMS(O) has RMS exactly
    0.2 whatever O is (any rank, any scale), and O and t O give the same
    step for t > 0."""
    r = _rng(11 + rank)
    U, _ = np.linalg.qr(r.standard_normal((shape[0], rank)))
    V, _ = np.linalg.qr(r.standard_normal((shape[1], rank)))
    O = U @ np.diag(r.uniform(0.1, 2.0, rank)) @ V.T
    W = r.normal(0, 0.02, shape)
    lr, wd = 1e-3, 0.1
    W1 = mo.apply_update(W, O, lr, wd, scaling="update_norm")
    upd = (W - W1) / lr - wd * W
    assert abs(math.sqrt(np.mean(upd ** 2)) - 0.2) < 1e-12
    W2 = mo.apply_update(W, 7.25 * O, lr, wd, scaling="update_norm")
    assert np.allclose(W1, W2, rtol=0, atol=1e-15)


def test_eq6_zero_update_is_decay_only():
    W = _rng(3).normal(0, 0.02, (8, 12))
    W1 = mo.apply_update(W, np.zeros_like(W), 1e-3, 0.1, scaling="update_norm")
    assert np.array_equal(W1, W - 1e-3 * (0.1 * W))


def test_eq6_full_step_rms():
    """Through the whole step: whatever N does to the singular values, the
    update-norm step moves W by exactly lr * 0.2 in RMS (plus the decay)."""
    r = _rng(41)
    W = r.normal(0, 0.02, (48, 96))
    G = r.normal(0, 1e-3, (48, 96))
    M = r.normal(0, 1e-3, (48, 96))
    for steps in (0, 1, 5):
        W1, _, X, rms = mo.muon_step(W, G, M, **dict(HYPER, ns_steps=steps), scaling="update_norm")
        upd = (W - W1) / HYPER["lr"] - HYPER["wd"] * W
        assert abs(math.sqrt(np.mean(upd ** 2)) - 0.2) < 1e-12
        assert abs(rms - math.sqrt(np.mean(X ** 2))) < 1e-15


# ---------------------------------------------------------------- momentum

def test_momentum_closed_form():
    r = _rng(31)
    G = r.standard_normal((5, 7))
    mu = 0.95
    M = np.zeros_like(G)
    for t in range(1, 5):
        M, N = mo.momentum_update(M, G, mu, nesterov=True)
        Mt = G * (1 - mu ** t) / (1 - mu)
        np.testing.assert_allclose(M, Mt, rtol=1e-13)
        np.testing.assert_allclose(N, mu * Mt + G, rtol=1e-13)
    M1, N1 = mo.momentum_update(np.zeros_like(G), G, mu, True)
    np.testing.assert_allclose(N1, 1.95 * G, rtol=1e-15)
    M1, N1 = mo.momentum_update(np.zeros_like(G), G, mu, False)
    np.testing.assert_array_equal(N1, G)


# ---------------------------------------------------------------- AdamW

def test_adamw_constant_gradient_closed_form():
    """Bias correction makes m_hat = g and v_hat = g^2 at every step under a
    constant gradient, so each step is ``W -= lr (g/(|g|+eps) + wd W)``."""
    r = _rng(41)
    W = r.normal(0, 0.02, 50)
    g = r.normal(0, 1e-3, 50)
    m = np.zeros(50)
    v = np.zeros(50)
    Wref = W.copy()
    lr, wd, eps = 1e-3, 0.1, 1e-8
    for t in range(1, 8):
        W, m, v = mo.adamw_step(W, g, m, v, lr=lr, wd=wd, t=t)
        Wref = Wref - lr * (g / (np.abs(g) + eps) + wd * Wref)
        np.testing.assert_allclose(W, Wref, rtol=1e-10)


def test_adamw_zero_grad_is_pure_decay():
    W = _rng(2).normal(0, 0.02, 20)
    z = np.zeros(20)
    W1, _, _ = mo.adamw_step(W, z, z, z, lr=1e-3, wd=0.1, t=1)
    np.testing.assert_allclose(W1, W - 1e-4 * W, rtol=4e-16, atol=0)


def test_adamw_brute_force():
    r = _rng(43)
    W, g = r.normal(0, 0.02, 33), r.normal(0, 1e-3, 33)
    m, v = r.normal(0, 1e-4, 33), np.abs(r.normal(0, 1e-7, 33))
    h = dict(lr=1e-3, wd=0.1, beta1=0.9, beta2=0.999, eps=1e-8, t=7)
    o = mo.adamw_step(W, g, m, v, **h)
    b = brute.adamw_step(W.tolist(), g.tolist(), m.tolist(), v.tolist(), **h)
    for x, y in zip(o, b):
        np.testing.assert_allclose(x, np.array(y), rtol=1e-13, atol=1e-20)


# ---------------------------------------------------------------- mutation check

def _pins_fail(muon_step_fn, orth_fn) -> bool:
    """Run a battery of the pins above against candidate functions; True if
    any of them detects a difference."""
    r = _rng(99)
    fails = []
    # closed form
    for shape in [(16, 48), (48, 16)]:
        N = r.standard_normal(shape)
        fails.append(sp.rel_fro(orth_fn(N, 5), sp.ns_closed_form(N, 5)) > 1e-9)
    # brute force on the full step (incl. momentum and apply)
    for shape in [(4, 8), (8, 4)]:
        W, G, M = r.normal(0, .02, shape), r.normal(0, 1, shape), r.normal(0, .5, shape)
        o = muon_step_fn(W, G, M, **HYPER)
        b = brute.muon_step(W.tolist(), G.tolist(), M.tolist(), **HYPER)
        fails.append(not np.allclose(o[0], np.array(b[0]), rtol=1e-10, atol=1e-14))
    # Lemma 1 scale through the full step
    Q = _orthonormal_rows(4, 8, 1)
    W = r.normal(0, .02, (4, 8))
    h = dict(HYPER, eps=0.0)
    W1 = muon_step_fn(W, Q / 1.95, np.zeros_like(W), **h)[0]
    upd = (W - W1) / h["lr"] - h["wd"] * W
    fx = _dec_map(Decimal("0.5"), 5)
    fails.append(abs(math.sqrt(np.mean(upd ** 2)) - 0.2 * fx) > 1e-9)
    return any(fails)


def _mk_orth(ns):
    def orth(N, steps):
        X0, _ = mo.frobenius_normalize(N, 1e-7)
        return ns(X0, steps, ABC)
    return orth


def _mk_step(ns=None, momentum=None, apply=None):
    def step(W, G, M, *, lr, wd, mu, nesterov, ns_steps, abc, rms_scale, eps):
        M1, N = (momentum or mo.momentum_update)(M, G, mu, nesterov)
        X0, _ = mo.frobenius_normalize(N, eps)
        X = (ns or mo.newton_schulz)(X0, ns_steps, abc)
        W1 = (apply or mo.apply_update)(W, X, lr, wd, rms_scale)
        return W1, M1, X, mo.update_rms(X)
    return step


def _ns_variant(flip_b=False, drop_c=False, drop_a=False, no_back_transpose=False):
    def ns(X0, steps, abc):
        a, b, c = abc
        b = -b if flip_b else b
        c = 0.0 if drop_c else c
        X = np.array(X0, dtype=np.float64)
        tall = X.shape[0] > X.shape[1]
        if tall:
            X = X.T
        for _ in range(steps):
            S = X @ X.T
            P = b * S + c * (S @ S)
            X = P @ X + (0.0 if drop_a else a) * X
        if no_back_transpose:
            return X.reshape(X0.shape)
        return X.T if tall else X
    return ns


@pytest.mark.filterwarnings("ignore::RuntimeWarning")
def test_mutants_are_caught():
    # the unmodified oracle passes every pin
    assert not _pins_fail(_mk_step(), _mk_orth(mo.newton_schulz))

    mutants = {
        "flip sign of b": _ns_variant(flip_b=True),
        "drop the c term": _ns_variant(drop_c=True),
        "drop the a term": _ns_variant(drop_a=True),
        "tall result reshaped, not transposed": _ns_variant(no_back_transpose=True),
    }
    for name, ns in mutants.items():
        assert _pins_fail(_mk_step(ns=ns), _mk_orth(ns)), name

    def momentum_old_buffer(M, G, mu, nesterov):     # Nesterov from stale M
        M = np.asarray(M, float)
        return mu * M + G, mu * M + G if nesterov else mu * M + G

    def apply_sqrt_min(W, X, lr, wd, s):
        return W - lr * (s * math.sqrt(min(W.shape)) * X + wd * W)

    def apply_decay_after(W, X, lr, wd, s):
        W1 = W - lr * s * math.sqrt(max(W.shape)) * X
        return W1 - lr * wd * W1

    def apply_no_scale(W, X, lr, wd, s):
        return W - lr * (X + wd * W)

    assert _pins_fail(_mk_step(momentum=momentum_old_buffer), _mk_orth(mo.newton_schulz))
    assert _pins_fail(_mk_step(apply=apply_sqrt_min), _mk_orth(mo.newton_schulz))
    assert _pins_fail(_mk_step(apply=apply_decay_after), _mk_orth(mo.newton_schulz))
    assert _pins_fail(_mk_step(apply=apply_no_scale), _mk_orth(mo.newton_schulz))


def _scaling_pins_fail(apply_fn):
    """The Eq. 5 / Eq. 6 pins above, run on a candidate apply_update."""
    r = _rng(77)
    fails = []
    W = r.normal(0, 0.02, (32, 96))
    O = sp.polar_factor(r.standard_normal((32, 96)))
    lr, wd = 1e-3, 0.1
    W1 = apply_fn(W, O, lr, wd, 0.2, "hidden", 300)
    upd = (W - W1) / lr - wd * W
    fails.append(abs(math.sqrt(np.mean(upd ** 2)) - 0.2 * math.sqrt(300 / 96)) > 1e-10)
    O2 = O[:, :] * np.linspace(0.2, 1.5, 96)[None, :]
    W1 = apply_fn(W, O2, lr, wd, 0.2, "update_norm", None)
    upd = (W - W1) / lr - wd * W
    fails.append(abs(math.sqrt(np.mean(upd ** 2)) - 0.2) > 1e-12)
    return any(fails)


def test_scaling_mutants_are_caught():
    assert not _scaling_pins_fail(mo.apply_update)

    def hidden_uses_shape(W, X, lr, wd, s, scaling, hidden):
        if scaling == "hidden":
            return mo.apply_update(W, X, lr, wd, s)
        return mo.apply_update(W, X, lr, wd, s, scaling, hidden)

    def norm_by_frobenius(W, X, lr, wd, s, scaling, hidden):   # ||O||_F instead of RMS(O)
        if scaling == "update_norm":
            return W - lr * (s * X / np.linalg.norm(X) + wd * W)
        return mo.apply_update(W, X, lr, wd, s, scaling, hidden)

    def norm_times_shape(W, X, lr, wd, s, scaling, hidden):    # Eq. 6 and Eq. 4 combined
        if scaling == "update_norm":
            return W - lr * (s * math.sqrt(max(W.shape)) * X / mo.update_rms(X) + wd * W)
        return mo.apply_update(W, X, lr, wd, s, scaling, hidden)

    for fn in (hidden_uses_shape, norm_by_frobenius, norm_times_shape):
        assert _scaling_pins_fail(fn), fn.__name__


def test_nonfinite_gradient_poisons_the_whole_update():
    """IEEE propagation (a reading: the pages say nothing): one NaN or Inf in
    G reaches ||N||_F, so X_N and the updated weight are NaN everywhere and
    the update RMS is NaN; the momentum is non-finite at that element only."""
    r = _rng(21)
    for v in (np.nan, np.inf, -np.inf):
        W = r.normal(0, 0.02, (6, 10))
        G = r.normal(0, 1e-3, (6, 10))
        G[2, 3] = v
        with np.errstate(invalid="ignore", over="ignore"):
            Wn, Mn, X, rms = mo.muon_step(W, G, np.zeros_like(W), **HYPER)
        assert np.isnan(Wn).all() and np.isnan(X).all() and math.isnan(rms)
        bad = ~np.isfinite(Mn)
        assert bad.sum() == 1 and bad[2, 3]
