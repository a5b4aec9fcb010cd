"""Seeded synthetic workloads for the Muon optimizer step.

This module holds shapes, dtypes, value distributions and seeds only -- none
of the optimizer's arithmetic -- so that both the HIP path (tests, bench) and
the fp64 oracle (tests) can be fed the very same tensors.  The optimizer's
own random numbers: there are none; every input is drawn here.

Shapes follow the pages' model families ("Muon is Scalable for LLM
Training": section 3.1 uses an 800M model whose MLP is a plain 2-layer
``[H, 4H]`` MLP; section 3.2 scales Llama-style dense models up to 1.5B
with GQA; section 3.4 and appendix F analyse a 64-expert MoE with MLA
projections and a router).  The exact layer counts and sizes are stated per
workload below.  Matrices of the same shape are carved out of one flat
buffer per tensor kind (weights, gradients, momenta) so that generation is
one RNG call per kind, and every view is 16-byte aligned.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional, Sequence, Tuple

import torch


@dataclasses.dataclass(frozen=True)
class MatGroup:
    """``count`` Muon matrices of shape ``[rows, cols]``."""
    name: str
    rows: int
    cols: int
    count: int


@dataclasses.dataclass(frozen=True)
class VecGroup:
    """``count`` AdamW tensors of shape ``shape`` (1-D norms, embeddings)."""
    name: str
    shape: Tuple[int, ...]
    count: int
    init: str = "normal"          # "normal" (N(0, w_std^2)) or "ones"


@dataclasses.dataclass(frozen=True)
class Workload:
    key: str
    description: str
    cid: int                       # seed namespace
    mats: Tuple[MatGroup, ...]
    vecs: Tuple[VecGroup, ...] = ()
    grad_dtype: torch.dtype = torch.bfloat16
    mom_dtype: torch.dtype = torch.bfloat16
    ns_dtype: torch.dtype = torch.bfloat16
    w_std: float = 0.02
    g_std: float = 1e-3
    # per-group gradient scale 10**U(-1, 1) for groups named "expert*",
    # one draw per expert shared by that expert's matrices
    expert_scale: bool = False
    experts_per_set: int = 0
    ns_steps: int = 5
    # the model's hidden size H (section 3.1, Eq. 5's 0.2 sqrt(H) scaling)
    hidden: int = 0
    lr: float = 1e-3
    wd: float = 0.1
    mu: float = 0.95
    steps: int = 1                 # number of steps with fresh gradients

    @property
    def n_mats(self) -> int:
        return sum(g.count for g in self.mats)

    @property
    def n_elems(self) -> int:
        return sum(g.rows * g.cols * g.count for g in self.mats)

    @property
    def n_vec_elems(self) -> int:
        return sum(math.prod(v.shape) * v.count for v in self.vecs)


def _dense800m() -> Workload:
    H, L = 1536, 24
    return Workload(
        key="dense800m",
        description=("800M-style dense decoder, 24 layers, H=1536: q/k/v/o "
                     "[1536,1536] and a 2-layer MLP [1536,6144]+[6144,1536] "
                     "per layer on Muon; 49 RMSNorm [1536] plus untied "
                     "embedding and LM head [32000,1536] on AdamW"),
        cid=2,
        mats=(MatGroup("attn_qkvo", H, H, 4 * L),
              MatGroup("mlp_up", H, 4 * H, L),
              MatGroup("mlp_down", 4 * H, H, L)),
        vecs=(VecGroup("rmsnorm", (H,), 2 * L + 1, init="ones"),
              VecGroup("embed", (32000, H), 1),
              VecGroup("lm_head", (32000, H), 1)),
        grad_dtype=torch.float32, mom_dtype=torch.bfloat16,
        ns_dtype=torch.bfloat16, hidden=H)


WORKLOADS: Dict[str, Workload] = {
    "fp32_128x512": Workload(
        key="fp32_128x512",
        description=("single fp32 matrix [128,512], W~N(0,0.02^2), 3 steps of "
                     "N(0,1) gradients from zero momentum"),
        cid=1, mats=(MatGroup("w", 128, 512, 1),),
        grad_dtype=torch.float32, mom_dtype=torch.float32,
        ns_dtype=torch.float32, g_std=1.0, steps=3, hidden=128),
    "dense800m": _dense800m(),
    "llama1p5b_gqa": Workload(
        key="llama1p5b_gqa",
        description=("Llama-style 1.5B dense with GQA, 24 layers, H=2048: "
                     "q/o [2048,2048], k/v [2048,512], SwiGLU gate/up "
                     "[2048,5632], down [5632,2048]"),
        cid=3,
        mats=(MatGroup("attn_qo", 2048, 2048, 48),
              MatGroup("attn_kv", 2048, 512, 48),
              MatGroup("mlp_gate_up", 2048, 5632, 48),
              MatGroup("mlp_down", 5632, 2048, 24)),
        grad_dtype=torch.bfloat16, mom_dtype=torch.bfloat16,
        ns_dtype=torch.bfloat16, hidden=2048),
    "moe_share": Workload(
        key="moe_share",
        description=("MoE block group, one GPU's share: 8 layers x 64 experts "
                     "x (gate [2048,1408], up [2048,1408], down [1408,2048]) "
                     "plus per-layer MLA-style [2048,512], [512,4096], "
                     "[2048,2048] and a router [2048,64]; expert gradients "
                     "scaled by 10**U(-1,1) per expert"),
        cid=4,
        mats=(MatGroup("expert_gate", 2048, 1408, 512),
              MatGroup("expert_up", 2048, 1408, 512),
              MatGroup("expert_down", 1408, 2048, 512),
              MatGroup("mla_down_kv", 2048, 512, 8),
              MatGroup("mla_up", 512, 4096, 8),
              MatGroup("attn_out", 2048, 2048, 8),
              MatGroup("router", 2048, 64, 8)),
        grad_dtype=torch.float32, mom_dtype=torch.bfloat16,
        ns_dtype=torch.bfloat16, expert_scale=True, experts_per_set=512, hidden=2048),
    "large_n5": Workload(
        key="large_n5",
        description=("large dense matrices: 16 x [8192,8192], 16 x "
                     "[8192,28672], 16 x [28672,8192], W~N(0,0.01^2), N=5"),
        cid=5,
        mats=(MatGroup("sq", 8192, 8192, 16),
              MatGroup("wide", 8192, 28672, 16),
              MatGroup("tall", 28672, 8192, 16)),
        grad_dtype=torch.bfloat16, mom_dtype=torch.bfloat16,
        ns_dtype=torch.bfloat16, w_std=0.01, hidden=8192),
    "kv_heads": Workload(
        key="kv_heads",
        description=("the 1.5B GQA model's attention with every head a separate "
                     "Muon matrix (head dim 128): 24 layers x (16 q, 4 k, 4 v "
                     "heads [2048,128] and 16 o heads [128,2048]) = 960 small "
                     "matrices"),
        cid=7,
        mats=(MatGroup("head_q", 2048, 128, 16 * 24),
              MatGroup("head_k", 2048, 128, 4 * 24),
              MatGroup("head_v", 2048, 128, 4 * 24),
              MatGroup("head_o", 128, 2048, 16 * 24)),
        grad_dtype=torch.bfloat16, mom_dtype=torch.bfloat16,
        ns_dtype=torch.bfloat16, hidden=2048),
}
WORKLOADS["large_n10"] = dataclasses.replace(
    WORKLOADS["large_n5"], key="large_n10", ns_steps=10, cid=6,
    description=WORKLOADS["large_n5"].description.replace("N=5", "N=10"))


def seed_of(cid: int, kind: int, step: int = 0) -> int:
    """Seed namespace: workload id, tensor kind (0 W, 1 G, 2 M, 3 scales,
    4 AdamW W, 5 AdamW g), step index."""
    return cid * 1_000_000 + kind * 10_000 + step


def _gen(device: torch.device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _normal_flat(n: int, std: float, dtype: torch.dtype, device, seed: int,
                 chunk: int = 1 << 28) -> torch.Tensor:
    """N(0, std^2) draws in fp32, cast to ``dtype`` (round-to-nearest-even)
    chunk by chunk so the fp32 staging stays bounded."""
    out = torch.empty(n, dtype=dtype, device=device)
    g = _gen(torch.device(device), seed)
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        out[s:e].copy_(torch.randn(e - s, generator=g, device=device,
                                   dtype=torch.float32).mul_(std))
    return out


@dataclasses.dataclass
class MuonTensors:
    """Caller-owned tensors of one workload's Muon matrices."""
    params: List[torch.Tensor]
    grads: List[torch.Tensor]
    moms: List[torch.Tensor]
    group_of: List[int]
    flats: Dict[str, torch.Tensor]


def _views(flat: torch.Tensor, shapes: Sequence[Tuple[int, int]]):
    out, off = [], 0
    for (r, c) in shapes:
        out.append(flat[off:off + r * c].view(r, c))
        off += r * c
    return out


def mat_shapes(wl: Workload) -> List[Tuple[int, int]]:
    return [(g.rows, g.cols) for g in wl.mats for _ in range(g.count)]


def expert_scales(wl: Workload, device="cpu") -> Optional[torch.Tensor]:
    """One gradient scale 10**U(-1,1) per expert (float32)."""
    if not wl.expert_scale:
        return None
    g = _gen(torch.device(device), seed_of(wl.cid, 3))
    u = torch.rand(wl.experts_per_set, generator=g, device=device,
                   dtype=torch.float32)
    return torch.pow(10.0, u * 2.0 - 1.0)


def make_grads(wl: Workload, device, step: int = 0,
               out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Flat gradient buffer for step ``step`` (fresh draw per step)."""
    n = wl.n_elems
    flat = _normal_flat(n, wl.g_std, wl.grad_dtype, device,
                        seed_of(wl.cid, 1, step))
    scales = expert_scales(wl, device)
    if scales is not None:
        off = 0
        for grp in wl.mats:
            sz = grp.rows * grp.cols
            if grp.name.startswith("expert"):
                blk = flat[off:off + sz * grp.count].view(grp.count, sz)
                blk.mul_(scales[:grp.count, None].to(blk.dtype))
            off += sz * grp.count
    if out is not None:
        out.copy_(flat)
        return out
    return flat


def make_muon_tensors(wl: Workload, device="cpu") -> MuonTensors:
    """Weights N(0, w_std^2) fp32, gradients of step 0, zero momentum
    (the momentum starts at the zero matrix, section 2.1)."""
    shapes = mat_shapes(wl)
    n = wl.n_elems
    W = _normal_flat(n, wl.w_std, torch.float32, device, seed_of(wl.cid, 0))
    G = make_grads(wl, device, 0)
    M = torch.zeros(n, dtype=wl.mom_dtype, device=device)
    group_of = [gi for gi, g in enumerate(wl.mats) for _ in range(g.count)]
    return MuonTensors(_views(W, shapes), _views(G, shapes), _views(M, shapes),
                       group_of, {"W": W, "G": G, "M": M})


@dataclasses.dataclass
class AdamWTensors:
    params: List[torch.Tensor]
    grads: List[torch.Tensor]
    m: List[torch.Tensor]
    v: List[torch.Tensor]


def make_adamw_tensors(wl: Workload, device="cpu",
                       grad_dtype: torch.dtype = torch.float32) -> AdamWTensors:
    """AdamW side tensors: RMSNorm gains = 1, others N(0, w_std^2); grads
    N(0, g_std^2); zero moments (step counter starts at 1)."""
    params, grads, ms, vs = [], [], [], []
    idx = 0
    for vg in wl.vecs:
        for _ in range(vg.count):
            numel = math.prod(vg.shape)
            if vg.init == "ones":
                p = torch.ones(numel, dtype=torch.float32, device=device)
            else:
                p = _normal_flat(numel, wl.w_std, torch.float32, device,
                                 seed_of(wl.cid, 4, idx))
            g = _normal_flat(numel, wl.g_std, grad_dtype, device,
                             seed_of(wl.cid, 5, idx))
            params.append(p.view(vg.shape))
            grads.append(g.view(vg.shape))
            ms.append(torch.zeros(vg.shape, dtype=torch.float32, device=device))
            vs.append(torch.zeros(vg.shape, dtype=torch.float32, device=device))
            idx += 1
    return AdamWTensors(params, grads, ms, vs)


def ns_flops(rows: int, cols: int, steps: int) -> Tuple[int, int]:
    """(algorithmic, dense) flop counts of ``steps`` Newton-Schulz iterations
    on one matrix: a symmetric product is counted once per distinct output
    entry (``3 m^2 n + m^3`` per iteration, m = min, n = max); dense counts
    every GEMM entry (``4 m^2 n + 2 m^3``)."""
    m, n = min(rows, cols), max(rows, cols)
    return steps * (3 * m * m * n + m ** 3), steps * (4 * m * m * n + 2 * m ** 3)


def workload_ns_flops(wl: Workload, steps: Optional[int] = None) -> Tuple[int, int]:
    s = wl.ns_steps if steps is None else steps
    alg = dense = 0
    for g in wl.mats:
        a, d = ns_flops(g.rows, g.cols, s)
        alg += a * g.count
        dense += d * g.count
    return alg, dense


def _bytes(dt: torch.dtype) -> int:
    return torch.empty((), dtype=dt).element_size()


def muon_elementwise_bytes_per_elem(wl: Workload) -> int:
    """Algorithmic HBM bytes per Muon element outside the GEMMs: read G,
    read + write M, write the Newton-Schulz input once, read + write W."""
    return (_bytes(wl.grad_dtype) + 2 * _bytes(wl.mom_dtype)
            + _bytes(wl.ns_dtype) + 8)


ADAMW_BYTES_PER_ELEM = 4 + 6 * 4   # g fp32; m, v, W read + write
