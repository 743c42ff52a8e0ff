"""Float64 CPU oracle for the gradients of exact attention.

TEST INFRASTRUCTURE ONLY (like oracle.attention): imported by the tests and the
benchmark's CPU-baseline leg, never by the HIP library.

The pages say what the backward pass keeps and recomputes (marketmaker.cc,
"Rückwärtsdurchlauf: Neu berechnen statt speichern": only O and the softmax
statistics are stored, the tiles of P are rebuilt from Q and K), but print no
gradient formulas. The gradients here are the derivatives of the definition in
oracle.attention (softmax(scale Q K^T) V with bottom-right causal masking and
grouped KV heads), by the chain rule through the row softmax:

  P = softmax(S), S = scale Q K^T (masked entries -inf, weight 0)
  dV = P^T dO
  dP = dO V^T
  dS_ij = P_ij (dP_ij - sum_k P_ik dP_ik)
  dQ = scale dS K,  dK = scale dS^T Q

with dK, dV of a KV head summed over the query heads that share it. Every
matrix is materialised in float64, P by the plain two-pass softmax; the row
term sum_k P_ik dP_ik is taken from its definition (not from O).
"""
from __future__ import annotations

import numpy as np


def _head_grads(q, k, v, do, causal: bool, scale: float):
    """Gradients of one head: q, do [N_q, d]; k, v [n, d]. Returns (dq, dk, dv)."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    do = np.asarray(do, np.float64)
    N_q, n = q.shape[0], k.shape[0]
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    if N_q == 0 or n == 0:
        return dq, dk, dv
    s = (q @ k.T) * float(scale)
    if causal:
        off = n - N_q
        masked = np.arange(n)[None, :] > (np.arange(N_q)[:, None] + off)
        s = np.where(masked, -np.inf, s)
    m = s.max(axis=1)
    empty = ~np.isfinite(m)
    m = np.where(empty, 0.0, m)
    e = np.exp(s - m[:, None])
    p = e / np.where(empty, 1.0, e.sum(axis=1))[:, None]
    p[empty] = 0.0
    dv = p.T @ do
    dp = do @ v.T
    ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
    dq = float(scale) * (ds @ k)
    dk = float(scale) * (ds.T @ q)
    return dq, dk, dv


def attention_backward_ref(q, k, v, do, causal: bool, scale: float):
    """Gradients of attention in float64.

    q, do: [B, H_q, N_q, d]; k, v: [B, H_kv, N_kv, d]. Returns (dq, dk, dv) as
    float64 arrays of the input shapes.
    """
    B, H_q, N_q, d = q.shape
    _, H_kv, N_kv, _ = k.shape
    if H_q % H_kv:
        raise ValueError("H_q must be a multiple of H_kv")
    G = H_q // H_kv
    dq = np.zeros((B, H_q, N_q, d))
    dk = np.zeros((B, H_kv, N_kv, d))
    dv = np.zeros((B, H_kv, N_kv, v.shape[3]))
    for b in range(B):
        for h in range(H_q):
            g = h // G
            a, bk, bv = _head_grads(q[b, h], k[b, g], v[b, g], do[b, h], causal, scale)
            dq[b, h] = a
            dk[b, g] += bk
            dv[b, g] += bv
    return dq, dk, dv


__all__ = ["attention_backward_ref"]
