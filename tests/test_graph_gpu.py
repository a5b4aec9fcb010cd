"""A plan's step captured in a HIP graph (torch.cuda.CUDAGraph) and
replayed: every replay must match the same step run eagerly, bit for bit
(the kernels are deterministic and take no host-side state that changes
between steps).  Replays are interleaved with unrelated eager work and
synchronisations, and each one is checked, since graph nodes that depend on
stale state show up only on replays after the first."""

from __future__ import annotations

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


def _state(seed, shapes, scale=1.0):
    g = torch.Generator(device=DEV).manual_seed(seed)
    P = [torch.randn(s, device=DEV, generator=g) * 0.02 for s in shapes]
    G = [torch.randn(s, device=DEV, generator=g) * 1e-3 * scale for s in shapes]
    M = [torch.zeros(s, device=DEV, dtype=torch.bfloat16) for s in shapes]
    return P, G, M


@pytest.mark.parametrize("scaling", ["shape", "update_norm"])
def test_plan_step_graph_replay(mod, scaling):
    # the 33 [96, 300] matrices (ragged W tiles) and the 32 [128, 256]
    # matrices (full W tiles, loaded ahead of the apply) take the fused
    # small-matrix kernel with the shape scaling (the update-norm scaling
    # runs them through the general kernels)
    shapes = [(300, 700), (700, 300), (512, 512), (1, 300)] + [(96, 300)] * 33 + [(128, 256)] * 32
    Pe, Ge, Me = _state(5, shapes)
    Pg, Gg, Mg = [t.clone() for t in Pe], [t.clone() for t in Ge], [t.clone() for t in Me]
    pe = mod.MuonPlan(Pe, Ge, Me)
    pg = mod.MuonPlan(Pg, Gg, Mg)
    ws_e = torch.empty(pe.workspace_bytes, dtype=torch.uint8, device=DEV)
    ws_g = torch.empty(pg.workspace_bytes, dtype=torch.uint8, device=DEV)
    rms_e = torch.zeros(len(shapes), device=DEV)
    rms_g = torch.zeros(len(shapes), device=DEV)
    kw = dict(HYP, scaling=scaling)

    # capture on a side stream after one eager warm-up step on each set
    pe.step(workspace=ws_e, update_rms=rms_e, **kw)
    pg.step(workspace=ws_g, update_rms=rms_g, **kw)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            pg.step(workspace=ws_g, update_rms=rms_g, **kw)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    # capture only records: the graph set is still one step in
    for a, b in zip(Pe, Pg):
        assert torch.equal(a, b)

    noise = torch.randn(1 << 20, device=DEV)
    for r in range(4):
        # new gradients each step, written in place (the graph reads them)
        for i, (ge, gg) in enumerate(zip(Ge, Gg)):
            fresh = torch.randn(ge.shape, device=DEV,
                                generator=torch.Generator(device=DEV).manual_seed(100 + 10 * r + i)) * 1e-3
            ge.copy_(fresh)
            gg.copy_(fresh)
        pe.step(workspace=ws_e, update_rms=rms_e, **kw)
        graph.replay()
        noise.mul_(1.0001).add_(0.5)          # unrelated eager work between replays
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(Pe, Pg)):
            assert torch.equal(a, b), (r, i, (a - b).abs().max().item())
        for a, b in zip(Me, Mg):
            assert torch.equal(a, b), r
        assert torch.equal(rms_e, rms_g), r
    pe.close()
    pg.close()
