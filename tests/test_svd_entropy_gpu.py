"""GPU parity of the SVD-entropy diagnostic (``mo_svd_entropy``) against the
fp64 oracle (section 3.4's entropy, appendix F's sorted singular values).

Tolerances come from the arithmetic: the fp64 Gram matrix of exact products
and the Householder reduction + bisection give each sigma_j^2 an absolute
error of a small multiple of (m + n) u sigma_1^2 (u = 2^-52); the test allows
eps = 8 (m + n) u, relative to sigma_1^2.  The entropy moves by at most about
m eps (1 + |ln eps|) / ln m under such a perturbation of the distribution.

Large sizes use signed, permuted Sylvester-Hadamard constructions
``H_m diag(s) P`` whose singular values are exactly ``sqrt(m) |s|``, so the
expected spectrum and entropy are known at any size without an SVD.
"""

from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import matrix_orthogonalizing_optimizer_amd as mo
from oracle import svd_entropy as se

pytestmark = pytest.mark.gpu

U = 2.0 ** -52


def _eps(r, c):
    return 8.0 * (r + c) * U


def _h_tol(r, c):
    m = min(r, c)
    e = _eps(r, c)
    return max(m * e * (1.0 + abs(math.log(e))) / max(math.log(m), 1.0), 1e-14)


def _gen(shape, seed, dtype, kind="gauss"):
    g = torch.Generator(device="cpu").manual_seed(seed)
    r, c = shape
    if kind == "gauss":
        x = torch.randn(r, c, generator=g)
    elif kind == "ill":                      # singular values spread over 1e-6 .. 1
        m = min(r, c)
        qa, _ = torch.linalg.qr(torch.randn(r, m, generator=g, dtype=torch.float64))
        qb, _ = torch.linalg.qr(torch.randn(c, m, generator=g, dtype=torch.float64))
        s = torch.logspace(0, -6, m, dtype=torch.float64)
        x = (qa * s) @ qb.T
    elif kind == "rank3":
        x = torch.randn(r, 3, generator=g) @ torch.randn(3, c, generator=g)
    elif kind == "zero":
        x = torch.zeros(r, c)
    else:
        raise ValueError(kind)
    return x.to(dtype).cuda()


def _check(x, h, sig):
    w = x.float().cpu().double().numpy()
    r, c = w.shape
    ref_s = se.singular_values(w)
    ref_h = se.entropy_from_sigma(ref_s)
    s1 = float(ref_s[0]) if ref_s.size else 0.0
    got = sig.cpu().numpy()
    assert got.shape == ref_s.shape
    assert np.all(np.diff(got) <= 0), "singular values not in decreasing order"
    err = np.max(np.abs(got ** 2 - ref_s ** 2)) if got.size else 0.0
    assert err <= _eps(r, c) * s1 * s1, (err, s1)
    assert abs(float(h) - ref_h) <= _h_tol(r, c), (float(h), ref_h)


SHAPES = [(1, 1), (1, 7), (7, 1), (2, 2), (2, 9), (3, 5), (5, 3), (63, 100), (64, 64),
          (65, 200), (200, 65), (130, 131), (129, 300), (300, 257)]


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("shape", SHAPES)
def test_svd_entropy_matches_oracle(shape, dtype):
    x = _gen(shape, 11 + shape[0] * 7 + shape[1], dtype)
    h, sig = mo.svd_entropy([x], sigma=True)
    torch.cuda.synchronize()
    _check(x, h[0], sig[0])


@pytest.mark.parametrize("kind", ["ill", "rank3", "zero"])
@pytest.mark.parametrize("shape", [(96, 160), (160, 96), (200, 200)])
def test_svd_entropy_special_spectra(shape, kind):
    x = _gen(shape, 5, torch.float32, kind)
    h, sig = mo.svd_entropy([x], sigma=True)
    torch.cuda.synchronize()
    _check(x, h[0], sig[0])
    if kind == "zero":
        assert float(h[0]) == 0.0 and torch.all(sig[0] == 0)
    if kind == "rank3":
        assert torch.all(sig[0][3:] <= 1e-5 * sig[0][0])


def test_svd_entropy_batch_and_workspace_independent():
    shapes = [(64, 100), (100, 64), (64, 64), (300, 129), (129, 300), (1, 5), (3, 3), (129, 129)]
    xs = [_gen(s, 100 + i, torch.float32) for i, s in enumerate(shapes)]
    h_all, s_all = mo.svd_entropy(xs, sigma=True)
    # one call per matrix
    for i, x in enumerate(xs):
        h1, s1 = mo.svd_entropy([x], sigma=True)
        assert torch.equal(h1[0], h_all[i]) and torch.equal(s1[0], s_all[i]), i
    # the smallest workspace (one matrix at a time) gives the same bits
    _, mn = mo.svd_entropy_workspace_size(tuple(x.shape) for x in xs)
    ws = torch.empty(mn, dtype=torch.uint8, device="cuda")
    h_min, s_min = mo.svd_entropy(xs, sigma=True, workspace=ws)
    assert torch.equal(h_min, h_all)
    for a, b in zip(s_min, s_all):
        assert torch.equal(a, b)
    for x, h, s in zip(xs, h_all, s_all):
        _check(x, h, s)


def _hadamard_gpu(m, n, s, seed, dtype):
    """[m, n] matrix H_m diag(s) on m of n columns, signed and permuted."""
    i = torch.arange(m, device="cuda")
    bits = i[:, None] & i[None, :]
    par = torch.zeros(m, m, dtype=torch.int64, device="cuda")
    while bool(bits.any()):
        par ^= bits & 1
        bits = bits >> 1
    h = (1 - 2 * par).to(torch.float32)
    g = torch.Generator(device="cpu").manual_seed(seed)
    w = torch.zeros(m, n, dtype=torch.float32, device="cuda")
    cols = torch.randperm(n, generator=g)[:m].cuda()
    signs = (torch.randint(0, 2, (m,), generator=g) * 2 - 1).to(torch.float32).cuda()
    w[:, cols] = h * (s.to(torch.float32).cuda() * signs)[None, :]
    return w.to(dtype)


@pytest.mark.parametrize("m,n,transpose", [(512, 512, False), (1024, 3000, True),
                                           (2048, 2048, False)])
def test_svd_entropy_hadamard_known_spectrum(m, n, transpose):
    g = torch.Generator(device="cpu").manual_seed(m + n)
    # bf16-exact magnitudes so that fp32 and bf16 inputs carry the same values
    s = (torch.randint(1, 256, (m,), generator=g).to(torch.float64) / 64.0)
    for dtype in (torch.float32, torch.bfloat16):
        w = _hadamard_gpu(m, n, s, m, dtype)
        if transpose:
            w = w.T.contiguous()
        h, sig = mo.svd_entropy([w], sigma=True)
        torch.cuda.synchronize()
        want_s = np.sort(math.sqrt(m) * s.numpy())[::-1]
        want_h = se.entropy_from_sigma(want_s)
        got = sig[0].cpu().numpy()
        s1 = want_s[0]
        assert np.max(np.abs(got ** 2 - want_s ** 2)) <= _eps(m, n) * s1 * s1
        assert abs(float(h[0]) - want_h) <= _h_tol(m, n), (float(h[0]), want_h)


def test_svd_entropy_max_size_hadamard():
    """m = 8192 (the largest min(rows, cols)), n = 8192: known spectrum."""
    m = n = 8192
    g = torch.Generator(device="cpu").manual_seed(8192)
    s = (torch.randint(1, 256, (m,), generator=g).to(torch.float64) / 64.0)
    w = _hadamard_gpu(m, n, s, 3, torch.bfloat16)
    h, sig = mo.svd_entropy([w], sigma=True)
    torch.cuda.synchronize()
    want_s = np.sort(math.sqrt(m) * s.numpy())[::-1]
    got = sig[0].cpu().numpy()
    s1 = want_s[0]
    assert np.max(np.abs(got ** 2 - want_s ** 2)) <= _eps(m, n) * s1 * s1
    assert abs(float(h[0]) - se.entropy_from_sigma(want_s)) <= _h_tol(m, n)


def test_svd_entropy_layer_shapes_against_oracle():
    """One attention and one MLP matrix of a 1536-wide layer, fp32 weights."""
    xs = [_gen((1536, 1536), 1, torch.float32), _gen((6144, 1536), 2, torch.float32)]
    h, sig = mo.svd_entropy(xs, sigma=True)
    torch.cuda.synchronize()
    for x, hh, ss in zip(xs, h, sig):
        _check(x, hh, ss)


@pytest.mark.parametrize("key", ["dense800m", "moe_share"])
def test_svd_entropy_full_workload(key):
    """The benchmark's launch configuration: one call over every Muon weight
    matrix of the workload (fp32 weights, full workspace).  Every matrix:
    singular values in decreasing order, entropy in [0, 1], and the trace
    identity sum sigma_i^2 = ||W||_F^2 (holds at any size).  One matrix per
    shape group against the oracle."""
    import workloads as W

    wl = W.WORKLOADS[key]
    T = W.make_muon_tensors(wl, torch.device("cuda"))
    mats = list(T.params)
    h, sig = mo.svd_entropy(mats, sigma=True)
    torch.cuda.synchronize()
    hh = h.cpu().numpy()
    assert np.all(hh >= 0.0) and np.all(hh <= 1.0 + 1e-12)
    for x, s in zip(mats, sig):
        r, c = x.shape
        s2 = s.cpu().numpy() ** 2
        assert np.all(np.diff(s2) <= 0.0)
        fro2 = float(torch.sum(x.double() ** 2))
        # each sigma_i^2 within eps sigma_1^2, so the sum within m eps sigma_1^2
        assert abs(float(np.sum(s2)) - fro2) <= min(r, c) * _eps(r, c) * float(s2[0]), (r, c)
    start = 0
    for g in wl.mats:
        i = start + g.count // 2
        _check(mats[i], h[i], sig[i])
        start += g.count
