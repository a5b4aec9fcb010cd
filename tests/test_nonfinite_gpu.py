"""NaN and Inf gradients (the pages say nothing; the library's contract is
IEEE propagation, see include/muon.h).

A NaN or an Inf anywhere in a matrix's gradient reaches its Frobenius norm,
so the whole Newton-Schulz iterate of that matrix -- and with it the whole
updated weight -- becomes NaN, and its reported update RMS is NaN: that RMS
is the per-matrix non-finite flag.  The momentum is elementwise, so only the
poisoned element is non-finite there.  Every other matrix of the same call
is computed exactly as if the poisoned ones were finite (bit for bit), on
both the general product kernels and the fused small-matrix kernel.  The
fp64 oracle behaves the same way (a CPU pin in test_oracle_pins.py).
"""

from __future__ import annotations

import math

import pytest
import torch

pytestmark = pytest.mark.gpu

DEV = "cuda"
HYP = dict(lr=1e-3, wd=0.1, mu=0.95, nesterov=True, ns_steps=5, rms_scale=0.2, eps=1e-7)


@pytest.fixture(scope="module")
def mod():
    import matrix_orthogonalizing_optimizer_amd as m
    m._lib.lib()
    return m


def _state(shapes, seed):
    g = torch.Generator().manual_seed(seed)
    Ps = [(torch.randn(*s, generator=g) * 0.02).to(DEV) for s in shapes]
    Gs = [(torch.randn(*s, generator=g) * 1e-3).to(DEV) for s in shapes]
    Ms = [torch.zeros(s, dtype=torch.bfloat16, device=DEV) for s in shapes]
    return Ps, Gs, Ms


# general kernels: 3 x [200, 456]; fused small-matrix kernel: 33 x [96, 300]
SHAPES = [(200, 456)] * 3 + [(456, 200)] + [(96, 300)] * 33
POISON = {0: (5, 7, math.nan), 1: (199, 455, math.inf), 3: (10, 3, -math.inf),
          4: (0, 0, math.nan), 5: (95, 299, math.inf)}


def test_nonfinite_gradient_poisons_its_matrix_only(mod):
    Ps, Gs, Ms = _state(SHAPES, 77)
    Pr, Gr, Mr = [p.clone() for p in Ps], [g.clone() for g in Gs], [m.clone() for m in Ms]
    for i, (r, c, v) in POISON.items():
        Gs[i][r, c] = v
    rms = torch.zeros(len(SHAPES), device=DEV)
    rms_r = torch.zeros(len(SHAPES), device=DEV)
    mod.muon_step(Ps, Gs, Ms, update_rms=rms, **HYP)
    mod.muon_step(Pr, Gr, Mr, update_rms=rms_r, **HYP)
    torch.cuda.synchronize()
    for i in range(len(SHAPES)):
        if i in POISON:
            r, c, v = POISON[i]
            assert torch.isnan(Ps[i]).all(), i
            assert math.isnan(rms[i].item()), i
            bad = ~torch.isfinite(Ms[i])
            assert bad.sum().item() == 1 and bool(bad[r, c]), i
            ok = torch.ones_like(bad)
            ok[r, c] = False
            assert torch.equal(Ms[i][ok], Mr[i][ok]), i
        else:
            assert torch.equal(Ps[i], Pr[i]), i
            assert torch.equal(Ms[i], Mr[i]), i
            assert rms[i].item() == rms_r[i].item() and math.isfinite(rms[i].item()), i
