"""Gradients of exact attention in fp64: the oracle for the backward kernels.

TEST INFRASTRUCTURE ONLY: the tests and the benchmark's CPU-baseline leg may
import this module; the product path never does.  It shares nothing with the
HIP library.

The pages do not spell out the backward pass.  They say that training
recomputes some quantities in the backward pass instead of storing them (the
paweldubiel.com FlashAttention note, "Mechanism and details"; the spicyshark.co
lesson, "Further reading": FlashAttention recomputes the scores).  The plainest
reading is the exact gradient of the forward's O = softmax(scale * Q K^T) V
(masked keys carry no weight) with respect to Q, K and V, which this module
writes out per (batch, query head) with the chain rule through the softmax:

    S  = scale * q k^T, masked keys -inf      P  = softmax(S) per row (max subtracted)
    O  = P v                                  D  = rowsum(dO * O) = rowsum(P * dP)
    dP = dO v^T                               dS = P * (dP - D)
    dq = scale * dS k                         dk = scale * dS^T q      dv = P^T dO

with k, v the rows of K/V head h / (Hq/Hkv); dk and dv of a K/V head sum the
contributions of every query head that reads it.  numpy float64 matmuls serve
as the library primitive; nothing is blocked or fused.
"""
from __future__ import annotations

import numpy as np


def _as_f64(x):
    if hasattr(x, "detach"):
        x = x.detach().to("cpu").double().numpy()
    return np.ascontiguousarray(x, dtype=np.float64)


def attention_backward(q, k, v, do, causal=False, scale=None):
    """q, do [B, Hq, N, d]; k, v [B, Hkv, N, d].

    Returns (dq [B, Hq, N, d], dk [B, Hkv, N, d], dv [B, Hkv, N, d],
    delta [B, Hq, N]) in float64, delta being D = rowsum(dO * O).
    """
    q, k, v, do = _as_f64(q), _as_f64(k), _as_f64(v), _as_f64(do)
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    if k.shape != (B, Hkv, N, d) or v.shape != k.shape or do.shape != q.shape or Hq % Hkv:
        raise ValueError("shapes: q, do [B, Hq, N, d]; k, v [B, Hkv, N, d]; Hq a multiple of Hkv")
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    G = Hq // Hkv
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    delta = np.zeros((B, Hq, N))
    masked = np.triu(np.ones((N, N), dtype=bool), 1) if causal else np.zeros((N, N), dtype=bool)
    for b in range(B):
        for h in range(Hq):
            hk = h // G
            kh, vh = k[b, hk], v[b, hk]
            s = scale * (q[b, h] @ kh.T)
            s[masked] = -np.inf
            m = s.max(axis=1, keepdims=True)
            e = np.exp(s - m)
            p = e / e.sum(axis=1, keepdims=True)
            o = p @ vh
            dp = do[b, h] @ vh.T
            dd = (do[b, h] * o).sum(axis=1)
            ds = p * (dp - dd[:, None])
            dq[b, h] = scale * (ds @ kh)
            dk[b, hk] += scale * (ds.T @ q[b, h])
            dv[b, hk] += p.T @ do[b, h]
            delta[b, h] = dd
    return dq, dk, dv, delta
