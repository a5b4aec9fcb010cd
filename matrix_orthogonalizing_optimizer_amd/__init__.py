"""MI355X-native Muon optimizer step (HIP, gfx950) behind a C ABI.

The method is that of "Muon is Scalable for LLM Training" (Moonshot AI /
UCLA, 2025): Nesterov momentum (section 2.1, Eq. 1), Frobenius
normalisation and quintic Newton-Schulz (Eq. 2), the 0.2 * sqrt(max(A, B))
shape scale with decoupled weight decay (section 2.2, Eq. 4), and AdamW with
the same learning rate and decay for non-matrix parameters.

This module only marshals torch tensors into the C ABI of ``libmuon.so``
(``include/muon.h``); PyTorch provides device memory and streams.  Every
arithmetic step runs in the HIP library, and there is no fallback.
"""

from __future__ import annotations

import ctypes
from typing import Iterable, List, Optional, Sequence, Tuple

import torch

from ._lib import (KERNEL_CLASS_NAMES, MO_BF16, MO_F32, MoMatrix, MoTensor,  # noqa: F401
                   MuonError, check, last_error, lib)

__all__ = ["muon_step", "adamw_step", "newton_schulz", "muon_workspace_size",
           "newton_schulz_workspace_size", "svd_entropy", "svd_entropy_workspace_size",
           "MuonPlan", "MuonAdamW", "profile_enable", "profile_read", "profile_reset",
           "MuonError", "KERNEL_CLASS_NAMES"]

_DT = {torch.float32: MO_F32, torch.bfloat16: MO_BF16}


def _dtype_code(dt: torch.dtype, what: str) -> int:
    if dt not in _DT:
        raise TypeError(f"{what}: dtype {dt} is not float32 or bfloat16")
    return _DT[dt]


def _common_dtype(ts: Sequence[torch.Tensor], what: str) -> torch.dtype:
    dts = {t.dtype for t in ts}
    if len(dts) != 1:
        raise TypeError(f"{what}: all tensors must share one dtype, got {dts}")
    return next(iter(dts))


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr()


def _stream_handle(device: torch.device, stream=None) -> int:
    if stream is None:
        return torch.cuda.current_stream(device).cuda_stream
    return getattr(stream, "cuda_stream", stream)


def _abc(abc) -> Optional[ctypes.Array]:
    if abc is None:
        return None
    a = (ctypes.c_float * 3)(*[float(x) for x in abc])
    return a


def _shape2(t: torch.Tensor) -> Tuple[int, int]:
    if t.dim() != 2:
        raise ValueError(f"Muon matrices must be 2-D, got shape {tuple(t.shape)}")
    return int(t.shape[0]), int(t.shape[1])


_WS: dict = {}


def _workspace(device: torch.device, nbytes: int, stream_handle: int) -> torch.Tensor:
    """A cached byte buffer of at least ``nbytes`` for one (device, stream).
    Calls queued on different streams never share it, and it is allocated on
    that stream, so torch's allocator orders any reuse of its memory after
    the work queued there."""
    key = (device.type, device.index, int(stream_handle or 0))
    ws = _WS.get(key)
    if ws is None or ws.numel() < nbytes:
        _WS.pop(key, None)
        n = max(nbytes, 256)
        if stream_handle and stream_handle != torch.cuda.current_stream(device).cuda_stream:
            with torch.cuda.stream(torch.cuda.ExternalStream(stream_handle, device=device)):
                ws = torch.empty(n, dtype=torch.uint8, device=device)
        else:
            ws = torch.empty(n, dtype=torch.uint8, device=device)
        _WS[key] = ws
    return ws


def _mk_tensors(params, grads, s0, s1=None):
    n = len(params)
    arr = (MoTensor * max(n, 1))()
    for i in range(n):
        r, c = (_shape2(params[i]) if params[i].dim() == 2
                else (1, params[i].numel()))
        arr[i].param = _ptr(params[i])
        arr[i].grad = _ptr(grads[i])
        arr[i].state0 = _ptr(s0[i])
        arr[i].state1 = _ptr(s1[i]) if s1 is not None else None
        arr[i].rows = r
        arr[i].cols = c
    return arr


def muon_workspace_size(shapes: Iterable[Tuple[int, int]],
                        ns_dtype: torch.dtype = torch.bfloat16) -> Tuple[int, int]:
    """(full, minimum) workspace bytes of ``mo_muon_step`` for these shapes."""
    shapes = list(shapes)
    arr = (MoTensor * max(len(shapes), 1))()
    for i, (r, c) in enumerate(shapes):
        arr[i].rows, arr[i].cols = int(r), int(c)
    full, mn = ctypes.c_size_t(), ctypes.c_size_t()
    check(lib().mo_muon_workspace_size(arr, len(shapes), _dtype_code(ns_dtype, "ns_dtype"),
                                       ctypes.byref(full), ctypes.byref(mn)))
    return full.value, mn.value


def muon_step(params: Sequence[torch.Tensor], grads: Sequence[torch.Tensor],
              moms: Sequence[torch.Tensor], *, lr: float, wd: float = 0.1,
              mu: float = 0.95, nesterov: bool = True, ns_steps: int = 5,
              abc=None, rms_scale: float = 0.2, eps: float = 1e-7,
              ns_dtype: torch.dtype = torch.bfloat16,
              update_rms: Optional[torch.Tensor] = None,
              workspace: Optional[torch.Tensor] = None, stream=None) -> None:
    """One Muon step over matrix parameters (``mo_muon_step``).

    ``params`` fp32 [A, B], ``grads`` fp32/bf16, ``moms`` fp32/bf16 (one
    dtype per list), all contiguous on one GPU.  ``update_rms``: optional
    fp32 tensor [len(params)] receiving sqrt(mean(X_N^2)) per matrix.
    """
    n = len(params)
    if not (len(grads) == len(moms) == n):
        raise ValueError("params, grads and moms must have the same length")
    if n == 0:
        return
    dev = params[0].device
    gdt = _dtype_code(_common_dtype(grads, "grads"), "grads")
    mdt = _dtype_code(_common_dtype(moms, "moms"), "moms")
    ndt = _dtype_code(ns_dtype, "ns_dtype")
    arr = _mk_tensors(params, grads, moms)
    full, mn = muon_workspace_size([_shape2(p) for p in params], ns_dtype)
    sh = _stream_handle(dev, stream)
    if workspace is None:
        workspace = _workspace(dev, full, sh)
    if update_rms is not None and (update_rms.dtype != torch.float32 or update_rms.numel() < n):
        raise ValueError("update_rms must be float32 with one slot per matrix")
    check(lib().mo_muon_step(arr, n, gdt, mdt, ndt, lr, wd, mu, int(nesterov), ns_steps,
                             _abc(abc), rms_scale, eps, _ptr(update_rms), _ptr(workspace),
                             workspace.numel() * workspace.element_size(),
                             sh))


_SCALINGS = {"shape": 0, "hidden": 1, "update_norm": 2}


class MuonPlan:
    """``mo_muon_plan_*``: binds one list of matrices for repeated steps."""

    def __init__(self, params: Sequence[torch.Tensor], grads: Sequence[torch.Tensor],
                 moms: Sequence[torch.Tensor], ns_dtype: torch.dtype = torch.bfloat16):
        n = len(params)
        if not (len(grads) == len(moms) == n):
            raise ValueError("params, grads and moms must have the same length")
        self.n = n
        self.device = params[0].device if n else torch.device("cuda")
        # the plan holds raw pointers: keep the tensors alive while it lives
        self._keep = (list(params), list(grads), list(moms))
        self._grad_meta = [(tuple(g.shape), g.dtype) for g in grads]
        self._grads_bound = True
        gdt = _dtype_code(_common_dtype(grads, "grads"), "grads") if n else MO_F32
        mdt = _dtype_code(_common_dtype(moms, "moms"), "moms") if n else MO_F32
        arr = _mk_tensors(params, grads, moms)
        h = ctypes.c_void_p()
        with torch.cuda.device(self.device):
            check(lib().mo_muon_plan_create(arr, n, gdt, mdt, _dtype_code(ns_dtype, "ns_dtype"),
                                            ctypes.byref(h)))
        self._h = h
        full, mn = ctypes.c_size_t(), ctypes.c_size_t()
        check(lib().mo_muon_plan_workspace_size(self._h, ctypes.byref(full), ctypes.byref(mn)))
        self.workspace_bytes, self.min_workspace_bytes = full.value, mn.value

    def step(self, *, lr: float, wd: float = 0.1, mu: float = 0.95, nesterov: bool = True,
             ns_steps: int = 5, abc=None, rms_scale: float = 0.2, eps: float = 1e-7,
             update_rms: Optional[torch.Tensor] = None,
             workspace: Optional[torch.Tensor] = None, stream=None,
             scaling: str = "shape", hidden: Optional[float] = None) -> None:
        """scaling: "shape" (0.2 sqrt(max(A, B)), Eq. 4 / 7), "hidden"
        (0.2 sqrt(hidden), Eq. 5) or "update_norm" (0.2 / RMS(X_N), Eq. 6)."""
        if self._h is None:
            raise RuntimeError("plan was closed")
        if not self._grads_bound:
            raise RuntimeError("gradients were released: call set_grads() before step()")
        if scaling not in _SCALINGS:
            raise ValueError(f"scaling must be one of {sorted(_SCALINGS)}")
        if scaling == "hidden" and hidden is None:
            raise ValueError('scaling="hidden" needs hidden=H')
        check(lib().mo_muon_plan_set_scaling(self._h, _SCALINGS[scaling],
                                             float(hidden) if hidden is not None else 0.0))
        sh = _stream_handle(self.device, stream)
        if workspace is None:
            workspace = _workspace(self.device, self.workspace_bytes, sh)
        check(lib().mo_muon_plan_step(self._h, lr, wd, mu, int(nesterov), ns_steps, _abc(abc),
                                      rms_scale, eps, _ptr(update_rms), _ptr(workspace),
                                      workspace.numel() * workspace.element_size(), sh))

    def set_grads(self, grads: Sequence[torch.Tensor], stream=None) -> None:
        """Rebind the plan's gradients (``mo_muon_plan_set_grads``): same
        shapes and dtype, new buffers.  Nothing is enqueued when the pointers
        are unchanged; otherwise one small kernel per 96 matrices updates the
        descriptor table on the stream, with no host synchronisation."""
        if self._h is None:
            raise RuntimeError("plan was closed")
        grads = list(grads)
        if len(grads) != self.n:
            raise ValueError(f"expected {self.n} gradients, got {len(grads)}")
        for i, (g, (shape, dt)) in enumerate(zip(grads, self._grad_meta)):
            if tuple(g.shape) != shape or g.dtype != dt:
                raise ValueError(f"grad {i}: expected {shape} {dt}, got {tuple(g.shape)} {g.dtype}")
        arr = (ctypes.c_void_p * max(self.n, 1))(*[_ptr(g) for g in grads])
        with torch.cuda.device(self.device):
            check(lib().mo_muon_plan_set_grads(self._h, arr, self.n,
                                               _stream_handle(self.device, stream)))
        self._keep = (self._keep[0], grads, self._keep[2])
        self._grads_bound = True

    def release_grads(self) -> None:
        """Drop the plan's references to its gradients once a step using
        them is queued (torch orders any reuse of their memory after the
        work already queued on the stream), so a framework that makes fresh
        gradients every step does not hold two sets.  The next step needs
        ``set_grads`` first."""
        self._keep = (self._keep[0], None, self._keep[2])
        self._grads_bound = False

    def close(self) -> None:
        if getattr(self, "_h", None) is not None:
            check(lib().mo_muon_plan_destroy(self._h))
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def adamw_step(params: Sequence[torch.Tensor], grads: Sequence[torch.Tensor],
               exp_avg: Sequence[torch.Tensor], exp_avg_sq: Sequence[torch.Tensor], *,
               lr: float, step: int, wd: float = 0.1, beta1: float = 0.9,
               beta2: float = 0.999, eps: float = 1e-8, stream=None) -> None:
    """AdamW for non-matrix parameters (``mo_adamw_step``); fp32 params and
    moments, fp32/bf16 grads, ``step`` >= 1."""
    n = len(params)
    if not (len(grads) == len(exp_avg) == len(exp_avg_sq) == n):
        raise ValueError("all lists must have the same length")
    if n == 0:
        return
    gdt = _dtype_code(_common_dtype(grads, "grads"), "grads")
    arr = (MoTensor * n)()
    for i in range(n):
        arr[i].param = _ptr(params[i])
        arr[i].grad = _ptr(grads[i])
        arr[i].state0 = _ptr(exp_avg[i])
        arr[i].state1 = _ptr(exp_avg_sq[i])
        arr[i].rows, arr[i].cols = 1, params[i].numel()
    check(lib().mo_adamw_step(arr, n, gdt, lr, wd, beta1, beta2, eps, int(step),
                              _stream_handle(params[0].device, stream)))


def newton_schulz_workspace_size(batch: int, rows: int, cols: int,
                                 dtype: torch.dtype = torch.bfloat16) -> int:
    out = ctypes.c_size_t()
    check(lib().mo_newton_schulz_workspace_size(batch, rows, cols, _dtype_code(dtype, "dtype"),
                                                ctypes.byref(out)))
    return out.value


def newton_schulz(x: torch.Tensor, *, ns_steps: int = 5, abc=None, eps: float = 1e-7,
                  out: Optional[torch.Tensor] = None,
                  workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Normalise and iterate Eq. 2 (``mo_newton_schulz``) on ``x`` [rows, cols]
    or [batch, rows, cols] (fp32 or bf16); returns X_N in x's dtype."""
    squeeze = x.dim() == 2
    x3 = x.unsqueeze(0) if squeeze else x
    if x3.dim() != 3:
        raise ValueError("x must be 2-D or 3-D")
    b, r, c = (int(v) for v in x3.shape)
    dt = _dtype_code(x.dtype, "x")
    if out is None:
        out = torch.empty_like(x3)
    ws_need = newton_schulz_workspace_size(b, r, c, x.dtype)
    sh = _stream_handle(x.device, stream)
    if workspace is None:
        workspace = _workspace(x.device, ws_need, sh)
    check(lib().mo_newton_schulz(_ptr(x3), _ptr(out), b, r, c, dt, ns_steps, _abc(abc), eps,
                                 _ptr(workspace), workspace.numel() * workspace.element_size(), sh))
    return out[0] if squeeze else out


def _mk_matrices(shapes_ptrs):
    n = len(shapes_ptrs)
    arr = (MoMatrix * max(n, 1))()
    for i, (ptr, r, c) in enumerate(shapes_ptrs):
        arr[i].data = ptr
        arr[i].rows = r
        arr[i].cols = c
    return arr


def svd_entropy_workspace_size(shapes: Iterable[Tuple[int, int]]) -> Tuple[int, int]:
    """(full, minimum) workspace bytes of ``mo_svd_entropy`` for [rows, cols] shapes."""
    shapes = list(shapes)
    arr = _mk_matrices([(16, r, c) for r, c in shapes])   # placeholder aligned address
    full, mn = ctypes.c_size_t(), ctypes.c_size_t()
    check(lib().mo_svd_entropy_workspace_size(arr, len(shapes), ctypes.byref(full),
                                              ctypes.byref(mn)))
    return full.value, mn.value


def svd_entropy(mats: Sequence[torch.Tensor], *, sigma: bool = False,
                workspace: Optional[torch.Tensor] = None, stream=None):
    """SVD entropy (section 3.4) of each 2-D matrix (fp32 or bf16, one dtype),
    as an fp64 tensor [len(mats)]; with ``sigma=True`` also a list of each
    matrix's singular values, largest first (appendix F), fp64."""
    mats = list(mats)
    if not mats:
        return (torch.empty(0, dtype=torch.float64), []) if sigma else torch.empty(0, dtype=torch.float64)
    dt = _dtype_code(_common_dtype(mats, "mats"), "mats")
    dev = mats[0].device
    arr = _mk_matrices([(_ptr(m),) + _shape2(m) for m in mats])
    ent = torch.empty(len(mats), dtype=torch.float64, device=dev)
    counts = [min(_shape2(m)) for m in mats]
    sig = torch.empty(sum(counts), dtype=torch.float64, device=dev) if sigma else None
    sh = _stream_handle(dev, stream)
    if workspace is None:
        full, _ = svd_entropy_workspace_size(_shape2(m) for m in mats)
        workspace = _workspace(dev, full, sh)
    check(lib().mo_svd_entropy(arr, len(mats), dt, _ptr(ent), _ptr(sig), _ptr(workspace),
                               workspace.numel() * workspace.element_size(), sh))
    if not sigma:
        return ent
    return ent, list(torch.split(sig, counts))


def profile_enable(classes: Iterable[str] = ()) -> None:
    """Time every later launch of the named kernel classes with HIP events."""
    mask = 0
    for c in classes:
        mask |= 1 << KERNEL_CLASS_NAMES.index(c)
    check(lib().mo_profile_enable(mask))


def profile_read(cls: str) -> Tuple[int, float, float]:
    """(launches, total GPU ms, total algorithmic work) of a kernel class."""
    n, ms, w = ctypes.c_int64(), ctypes.c_double(), ctypes.c_double()
    check(lib().mo_profile_read(KERNEL_CLASS_NAMES.index(cls), ctypes.byref(n),
                                ctypes.byref(ms), ctypes.byref(w)))
    return n.value, ms.value, w.value


def profile_reset() -> None:
    check(lib().mo_profile_reset())


class MuonAdamW:
    """Optimizer front: 2-D parameters take the Muon step, everything else
    (RMSNorm gains, embeddings and LM head passed in ``adamw_params``) takes
    AdamW, with one shared learning rate and weight decay (section 2.2).

    State lives in torch tensors owned here (momentum per Muon matrix; m, v
    per AdamW tensor), so checkpointing is saving ``state_dict()``.
    """

    def __init__(self, muon_params: Sequence[torch.Tensor],
                 adamw_params: Sequence[torch.Tensor] = (), *, lr: float = 1e-3,
                 wd: float = 0.1, mu: float = 0.95, nesterov: bool = True,
                 ns_steps: int = 5, mom_dtype: torch.dtype = torch.bfloat16,
                 ns_dtype: torch.dtype = torch.bfloat16, betas=(0.9, 0.999),
                 adam_eps: float = 1e-8):
        self.muon_params: List[torch.Tensor] = list(muon_params)
        self.adamw_params: List[torch.Tensor] = list(adamw_params)
        for p in self.muon_params:
            _shape2(p)
        self.lr, self.wd, self.mu, self.nesterov = lr, wd, mu, nesterov
        self.ns_steps, self.ns_dtype, self.betas, self.adam_eps = ns_steps, ns_dtype, betas, adam_eps
        self.momentum = [torch.zeros_like(p, dtype=mom_dtype) for p in self.muon_params]
        self.exp_avg = [torch.zeros_like(p, dtype=torch.float32) for p in self.adamw_params]
        self.exp_avg_sq = [torch.zeros_like(p, dtype=torch.float32) for p in self.adamw_params]
        self.t = 0
        self._plan: Optional[MuonPlan] = None
        self.plans_created = 0

    def _grads(self, ps):
        gs = [p.grad for p in ps]
        if any(g is None for g in gs):
            raise RuntimeError("every parameter needs a gradient before step()")
        return gs

    def zero_grad(self, set_to_none: bool = True) -> None:
        """As ``torch.optim.Optimizer.zero_grad``: drop (or zero) every
        parameter's gradient."""
        for p in self.muon_params + self.adamw_params:
            if p.grad is None:
                continue
            if set_to_none:
                p.grad = None
            else:
                p.grad.zero_()

    def step(self, lr: Optional[float] = None, update_rms: Optional[torch.Tensor] = None) -> None:
        lr = self.lr if lr is None else lr
        self.t += 1
        if self.muon_params:
            gs = self._grads(self.muon_params)
            if self._plan is None:
                # the plan binds params and momenta once; gradients that move
                # between steps (zero_grad(set_to_none=True)) are rebound
                self._plan = MuonPlan(self.muon_params, gs, self.momentum, self.ns_dtype)
                self.plans_created += 1
            else:
                self._plan.set_grads(gs)
            self._plan.step(lr=lr, wd=self.wd, mu=self.mu, nesterov=self.nesterov,
                            ns_steps=self.ns_steps, update_rms=update_rms)
            self._plan.release_grads()
        if self.adamw_params:
            adamw_step(self.adamw_params, self._grads(self.adamw_params), self.exp_avg,
                       self.exp_avg_sq, lr=lr, step=self.t, wd=self.wd, beta1=self.betas[0],
                       beta2=self.betas[1], eps=self.adam_eps)

    def state_dict(self) -> dict:
        return {"t": self.t, "momentum": [m.clone() for m in self.momentum],
                "exp_avg": [m.clone() for m in self.exp_avg],
                "exp_avg_sq": [v.clone() for v in self.exp_avg_sq]}

    def load_state_dict(self, sd: dict) -> None:
        # checked in full before anything is copied
        for name in ("momentum", "exp_avg", "exp_avg_sq"):
            dst, src = getattr(self, name), sd[name]
            if len(src) != len(dst):
                raise ValueError(f"state_dict[{name!r}] has {len(src)} tensors, the optimizer {len(dst)}")
            for i, (d, t) in enumerate(zip(dst, src)):
                if tuple(t.shape) != tuple(d.shape):
                    raise ValueError(f"state_dict[{name!r}][{i}] has shape {tuple(t.shape)}, "
                                     f"expected {tuple(d.shape)}")
        self.t = int(sd["t"])
        for name in ("momentum", "exp_avg", "exp_avg_sq"):
            for d, t in zip(getattr(self, name), sd[name]):
                d.copy_(t)
