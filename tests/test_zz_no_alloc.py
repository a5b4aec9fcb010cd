"""``mo_muon_step_noalloc`` (the step with the library's own scratch, for
callers that cannot allocate) against ``mo_muon_step`` through the C ABI.

Two calls in a row, the second on smaller matrices, each on a copy of the
same state that ``mo_muon_step`` gets: parameters, momenta and update RMS
must match bit for bit (results do not depend on the workspace, and the
scratch keeps the first call's contents when the second starts).  The first
set mixes shape groups, both orientations and a group of small matrices
(the fused kernel); at 256 MiB of scratch its groups run in chunks.  A set
that needs more than the scratch is rejected before anything changes.
"""

from __future__ import annotations

import ctypes

import pytest
import torch

pytestmark = pytest.mark.gpu

DEV = "cuda"
LR, WD, MU, NS, SCALE, EPS = 1e-3, 0.1, 0.95, 5, 0.2, 1e-7


@pytest.fixture(scope="module")
def L():
    from matrix_orthogonalizing_optimizer_amd import _lib
    return _lib


def _state(shapes, seed, gdt=torch.float32):
    g = torch.Generator().manual_seed(seed)
    P = [(torch.randn(*s, generator=g) * 0.02).to(DEV) for s in shapes]
    G = [(torch.randn(*s, generator=g) * 1e-3).to(gdt).to(DEV) for s in shapes]
    M = [(torch.randn(*s, generator=g) * 1e-3).to(torch.bfloat16).to(DEV) for s in shapes]
    return P, G, M


def _arr(L, P, G, M):
    arr = (L.MoTensor * len(P))()
    for i, (p, g, m) in enumerate(zip(P, G, M)):
        arr[i].param, arr[i].grad, arr[i].state0 = p.data_ptr(), g.data_ptr(), m.data_ptr()
        arr[i].state1 = None
        arr[i].rows, arr[i].cols = p.shape
    return arr


def _both(L, shapes, seed, gdt):
    P, G, M = _state(shapes, seed, gdt)
    Pn, Mn = [p.clone() for p in P], [m.clone() for m in M]
    n = len(shapes)
    gcode = L.MO_F32 if gdt == torch.float32 else L.MO_BF16
    rms = torch.zeros(n, device=DEV)
    rms_n = torch.full((n,), -1.0, device=DEV)
    stream = torch.cuda.current_stream().cuda_stream
    full, mn = ctypes.c_size_t(), ctypes.c_size_t()
    arr = _arr(L, P, G, M)
    L.check(L.lib().mo_muon_workspace_size(arr, n, L.MO_BF16, ctypes.byref(full), ctypes.byref(mn)))
    ws = torch.empty(full.value, dtype=torch.uint8, device=DEV)
    L.check(L.lib().mo_muon_step(arr, n, gcode, L.MO_BF16, L.MO_BF16, LR, WD, MU, 1, NS, None, SCALE, EPS,
                                 rms.data_ptr(), ws.data_ptr(), full.value, stream))
    L.check(L.lib().mo_muon_step_noalloc(_arr(L, Pn, G, Mn), n, gcode, L.MO_BF16, L.MO_BF16, LR, WD, MU, 1, NS,
                                         None, SCALE, EPS, rms_n.data_ptr(), stream))
    torch.cuda.synchronize()
    for a, b in zip(P + M, Pn + Mn):
        assert torch.equal(a, b)
    assert torch.equal(rms, rms_n)
    return full.value


def test_noalloc_matches_workspace_step_twice(L):
    big = [(1536, 6144)] * 3 + [(6144, 1536)] * 3 + [(1536, 1536)] * 2 + [(300, 700), (700, 300)] + \
        [(96, 300)] * 40
    full = _both(L, big, 10, torch.float32)
    assert full > (256 << 20)                     # the first call runs in chunks
    _both(L, [(256, 512), (512, 256), (130, 70)], 20, torch.bfloat16)


def test_noalloc_rejects_what_does_not_fit(L):
    shapes = [(8192, 8192)]                        # one matrix needs > 256 MiB
    P, G, M = _state(shapes, 30)
    P0, M0 = [p.clone() for p in P], [m.clone() for m in M]
    rc = L.lib().mo_muon_step_noalloc(_arr(L, P, G, M), 1, L.MO_F32, L.MO_BF16, L.MO_BF16, LR, WD, MU, 1, NS,
                                      None, SCALE, EPS, None, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert rc == L.MO_EWORKSPACE
    assert "scratch" in L.last_error()
    assert torch.equal(P[0], P0[0]) and torch.equal(M[0], M0[0])
