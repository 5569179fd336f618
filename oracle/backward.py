"""Gradients of exact attention: the oracle of the backward kernels.

TEST INFRASTRUCTURE ONLY (see the package docstring): never imported by the
product path.  No code is shared with the HIP kernels.

What it computes.  "Flash Attention và IO" asks for the backward pass to be
timed beside the forward when the goal is training (section "Kernel đúng còn
phải hợp với tải") and for an implementation's gradients, not only its
outputs, to be compared with another one's at thresholds suited to the dtype
(section "Bài tập kiểm tính đúng trước khi đo tốc độ"); FLAMIA's training
timings are forward plus backward.  The pages print no backward formulas, so
the oracle is the definition: the derivatives of O = softmax(scale Q K^T + mask) V
(the forward of oracle.exact) with respect to Q, K and V, for an upstream
gradient dO, written out by the chain rule in float64 for each (sequence,
head):

    P  = softmax(S),  S = scale Q K^T + mask   (masked entries: P = 0)
    dV = P^T dO
    dP = dO V^T
    D  = rowsum(P * dP)  (= rowsum(dO * O))
    dS = P * (dP - D)    (the softmax Jacobian applied row by row)
    dQ = scale dS K,     dK = scale dS^T Q.

A row with no visible key has O = 0 and contributes nothing.  Layouts as
oracle.exact.attention: [B, N, H, d], or [N_total, H, d] with host cu_seqlens.
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np


def _sequence_grads(q, k, v, do, scale: float, causal: bool):
    """dQ, dK, dV of one (sequence, head): q, k [n, d], v, do [n, dv]."""
    n = q.shape[0]
    s = float(scale) * (q @ k.T)
    if causal:
        s = np.where(np.arange(n)[None, :] > np.arange(n)[:, None], -np.inf, s)
    m = s.max(axis=1, keepdims=True)
    m = np.where(np.isfinite(m), m, 0.0)
    p = np.exp(s - m)
    l = p.sum(axis=1, keepdims=True)
    p = np.divide(p, l, out=np.zeros_like(p), where=l > 0)
    dv = p.T @ do
    dp = do @ v.T
    dd = (p * dp).sum(axis=1, keepdims=True)
    ds = p * (dp - dd)
    dq = float(scale) * (ds @ k)
    dk = float(scale) * (ds.T @ q)
    return dq, dk, dv


def attention_grads(q, k, v, do, scale: float, causal: bool = False,
                    cu_seqlens: Optional[Sequence[int]] = None):
    """Returns (dQ, dK, dV) in float64, each shaped like its input."""
    q, k, v, do = (np.asarray(a, dtype=np.float64) for a in (q, k, v, do))
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    if cu_seqlens is not None:
        cu = [int(x) for x in cu_seqlens]
        for doc in range(len(cu) - 1):
            a, b = cu[doc], cu[doc + 1]
            if b <= a:
                continue
            for h in range(q.shape[1]):
                dq[a:b, h], dk[a:b, h], dv[a:b, h] = _sequence_grads(
                    q[a:b, h], k[a:b, h], v[a:b, h], do[a:b, h], scale, causal)
        return dq, dk, dv
    B, N, H, _ = q.shape
    for b in range(B):
        for h in range(H):
            dq[b, :, h], dk[b, :, h], dv[b, :, h] = _sequence_grads(
                q[b, :, h], k[b, :, h], v[b, :, h], do[b, :, h], scale, causal)
    return dq, dk, dv


def row_dot(o, do) -> np.ndarray:
    """D = rowsum(dO * O) per (sequence or document, head, row), laid out as
    the LSE: [B, H, N] for [B, N, H, d] inputs, [H, N_total] for packed."""
    o, do = np.asarray(o, dtype=np.float64), np.asarray(do, dtype=np.float64)
    d = (o * do).sum(axis=-1)
    return d.transpose(0, 2, 1) if d.ndim == 3 else d.T


def grads_at(q, k, v, do, scale: float, causal: bool, q_rows, k_rows, chunk: int = 1024):
    """The same gradients for selected rows of one (sequence, head), without
    an n x n matrix: q, k [n, d], v, do [n, dv] (float64-exact values).

    L_i = logsumexp_j S_ij and D_i = rowsum(dO_i * O_i) are formed for every
    row, ``chunk`` rows at a time; then dQ at q_rows from P_i. and dP_i., and
    dK, dV at k_rows from the columns P_.j (every query that sees key j).
    Returns (dq [len(q_rows), d], dk [len(k_rows), d], dv [len(k_rows), dv],
    parts), parts holding L, D and O for every row (for error bounds)."""
    q, k, v, do = (np.asarray(a, dtype=np.float64) for a in (q, k, v, do))
    n = q.shape[0]
    L = np.empty(n)
    O = np.empty((n, v.shape[1]))
    for a in range(0, n, chunk):
        b = min(n, a + chunk)
        s = float(scale) * (q[a:b] @ k.T)
        if causal:
            s = np.where(np.arange(n)[None, :] > np.arange(a, b)[:, None], -np.inf, s)
        m = s.max(axis=1, keepdims=True)
        p = np.exp(s - m)
        l = p.sum(axis=1, keepdims=True)
        L[a:b] = (m + np.log(l))[:, 0]
        O[a:b] = (p / l) @ v
    D = (O * do).sum(axis=1)
    qr = np.asarray(q_rows, dtype=np.int64)
    kr = np.asarray(k_rows, dtype=np.int64)
    # dQ rows
    s = float(scale) * (q[qr] @ k.T)
    if causal:
        s = np.where(np.arange(n)[None, :] > qr[:, None], -np.inf, s)
    p = np.exp(s - L[qr][:, None])
    dp = do[qr] @ v.T
    dq = float(scale) * ((p * (dp - D[qr][:, None])) @ k)
    # dK, dV columns: every query row i against key j
    s = float(scale) * (q @ k[kr].T)                      # [n, len(k_rows)]
    if causal:
        s = np.where(kr[None, :] > np.arange(n)[:, None], -np.inf, s)
    p = np.exp(s - L[:, None])
    dp = do @ v[kr].T
    dk = float(scale) * ((p * (dp - D[:, None])).T @ q)
    dv = p.T @ do
    return dq, dk, dv, {"L": L, "D": D, "O": O}
