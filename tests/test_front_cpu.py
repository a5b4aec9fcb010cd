"""Host-side behaviour of the optimizer front (no GPU): the state-dict round
trip of ``MuonAdamW`` and its refusal of mismatched checkpoints, checked in
full before anything is overwritten."""

from __future__ import annotations

import pytest
import torch

import matrix_orthogonalizing_optimizer_amd as mo


def _opt():
    ps = [torch.zeros(8, 16), torch.zeros(16, 4)]
    vs = [torch.zeros(16)]
    return mo.MuonAdamW(ps, vs)


def test_state_dict_round_trip():
    a, b = _opt(), _opt()
    a.t = 7
    for i, m in enumerate(a.momentum + a.exp_avg + a.exp_avg_sq):
        m.fill_(float(i + 1))
    b.load_state_dict(a.state_dict())
    assert b.t == 7
    for x, y in zip(a.momentum + a.exp_avg + a.exp_avg_sq, b.momentum + b.exp_avg + b.exp_avg_sq):
        assert torch.equal(x, y)


@pytest.mark.parametrize("bad", ["count", "shape"])
def test_mismatched_state_dict_is_refused_untouched(bad):
    a, b = _opt(), _opt()
    sd = a.state_dict()
    for m in sd["momentum"]:
        m.fill_(3.0)
    if bad == "count":
        sd["exp_avg_sq"] = []
    else:
        sd["exp_avg"][0] = torch.zeros(15)
    b.t = 2
    with pytest.raises(ValueError):
        b.load_state_dict(sd)
    assert b.t == 2
    assert all(float(m.abs().sum()) == 0.0 for m in b.momentum)
