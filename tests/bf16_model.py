"""A CPU model of where the bf16 Newton-Schulz path rounds.

Test infrastructure: it backs the tolerance statements of the bf16 parity
tests (which shapes and step counts reach which error) with committed code.
It imitates the GPU path's rounding points, not its code:

* X_0 is N stored in bf16 (round to nearest even), unscaled; the scale
  r = 1 / (||N||_F + eps) comes from N before rounding, in double;
* every product accumulates in fp32 (numpy float32 matmul) on operands
  that are exact bf16 values;
* S = bf16(s X X^T) with s = r^2 on the first iteration, else 1;
* P' = bf16(c S S + b S + a I) -- the linear term folded into P', as the
  kernels do;
* X' = bf16(s P' X) with s = r on the first iteration; the last iterate
  stays fp32;
* a tall matrix is processed as its transpose.

The summation order differs from the matrix cores', so the model matches the
GPU's error statistically (same magnitude, same dependence on shape and N),
not digit for digit.

``ns_gram_space`` models the fused small-matrix path instead (m <= 128,
N <= 5), which iterates on the m x m Gram matrix at about fp32 precision.
"""

from __future__ import annotations

import numpy as np


def to_bf16(x) -> np.ndarray:
    """fp32 -> nearest-even bf16, returned as float32 holding that value."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    u = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) & np.uint32(0xFFFF0000)
    return u.view(np.float32)


def ns_bf16(N, steps: int, abc=(3.4445, -4.7750, 2.0315), eps: float = 1e-7,
            rounding: bool = True) -> np.ndarray:
    """X_N of the bf16 path for one Newton-Schulz input N (float64 or float32).
    ``rounding=False`` keeps every stored value in fp32 (the model's own
    sanity check: it must then agree with the fp64 oracle to fp32 accuracy)."""
    N64 = np.asarray(N, dtype=np.float64)
    tall = N64.shape[0] > N64.shape[1]
    if tall:
        N64 = N64.T
    a, b, c = (np.float32(v) for v in abc)
    rnd = to_bf16 if rounding else (lambda v: np.asarray(v, dtype=np.float32))
    r = np.float32(1.0 / (np.sqrt(np.sum(N64 * N64)) + eps))
    X = rnd(N64.astype(np.float32))
    m = X.shape[0]
    eye = np.eye(m, dtype=np.float32)
    for k in range(steps):
        s2 = r * r if k == 0 else np.float32(1.0)
        S = rnd((X @ X.T) * s2)
        P = rnd(c * (S @ S) + b * S + a * eye)
        Y = (P @ X) * (r if k == 0 else np.float32(1.0))
        X = Y if k + 1 == steps else rnd(Y)
    if steps == 0:
        X = X * r
    X = X.astype(np.float64)
    return X.T if tall else X


def nesterov_input_fp32(M, G, mu: float = 0.95) -> np.ndarray:
    """N = mu (mu M + G) + G evaluated in fp32 (the momentum kernel's
    arithmetic) from the stored momentum and gradient."""
    M32 = np.asarray(M, dtype=np.float32)
    G32 = np.asarray(G, dtype=np.float32)
    mu32 = np.float32(mu)
    Mn = mu32 * M32 + G32
    return (mu32 * Mn + G32).astype(np.float64)


def split_bf16(A):
    """A = hi + lo with hi = bf16(A), lo = bf16(A - hi) (fp32 arithmetic)."""
    A32 = np.asarray(A, dtype=np.float32)
    hi = to_bf16(A32)
    lo = to_bf16((A32 - hi).astype(np.float32))
    return hi, lo


def matmul_split3(A, B) -> np.ndarray:
    """A B as three bf16 products of split operands, Ah Bh + Ah Bl + Al Bh,
    accumulated in fp32."""
    Ah, Al = split_bf16(A)
    Bh, Bl = split_bf16(B)
    return (Ah @ Bh + Ah @ Bl + Al @ Bh).astype(np.float32)


def ns_gram_space(N, steps: int, abc=(3.4445, -4.7750, 2.0315), eps: float = 1e-7) -> np.ndarray:
    """X_N of the fused small-matrix path (m <= 128): the iteration carried
    out on m x m matrices,
        S_0 = r^2 X_0 X_0^T,  P_k = a I + b S_k + c S_k^2,
        S_{k+1} = P_k S_k P_k,  Q_{k+1} = P_k Q_k,  X_N = r Q_N X_0,
    with X_0 = bf16(N) unscaled, S_0 accumulated in fp32, every m x m
    product three bf16 products of split operands (fp32 accumulation),
    S, P, Q held in fp32, and X_N = r X_0^T (Q_hi + Q_lo) transposed.  A
    tall matrix is processed as its transpose.  steps >= 1."""
    N64 = np.asarray(N, dtype=np.float64)
    tall = N64.shape[0] > N64.shape[1]
    if tall:
        N64 = N64.T
    a, b, c = (np.float32(v) for v in abc)
    r = np.float32(1.0 / (np.sqrt(np.sum(N64 * N64)) + eps))
    X0 = to_bf16(N64.astype(np.float32))
    S = (X0 @ X0.T).astype(np.float32) * (r * r)
    eye = np.eye(S.shape[0], dtype=np.float32)
    Q = None
    for k in range(steps):
        P = (c * matmul_split3(S, S) + b * S + a * eye).astype(np.float32)
        if k + 1 < steps:
            S = matmul_split3(P, matmul_split3(S, P))
        Q = P if Q is None else matmul_split3(P, Q)
    Qh, Ql = split_bf16(Q)
    X = ((X0.T @ Qh + X0.T @ Ql).T * r).astype(np.float64)
    return X.T if tall else X
