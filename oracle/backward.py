"""Gradients of softmax attention, in float64, by the definition.

TEST INFRASTRUCTURE ONLY (see the package docstring): imported by the tests,
never by the product path, and sharing no code with it.

The pages present FlashAttention as a way to speed up the *training* of large
models ("FlashAttention-3 (PT)", introduction and section "Desempenho e
importancia"; "Flash Attention" glossary page, third paragraph and section
"Exemplo"), which needs the backward pass, but they print no formula for it.
What is computed here is therefore the plain chain rule through the forward
definition of ``oracle.attention``, for the loss L = sum(dO * O) (so dQ, dK, dV
are the vector-Jacobian products with the upstream gradient dO).

Per (b, h), with S = scale * Q K^T (masked entries -inf) and P = softmax(S)
row by row, O = P V:
  dV = P^T dO                                (O is linear in V)
  dP = dO V^T                                (O is linear in P)
  dS_ij = P_ij * (dP_ij - sum_l P_il dP_il)  (Jacobian of each softmax row)
  dQ = scale * dS K,   dK = scale * dS^T Q   (S is bilinear in Q and K)
Masked entries have P = 0, hence dS = 0.  Full rows of S and P are formed,
a band of complete rows at a time.
"""
from __future__ import annotations

import numpy as np


def _f64(x) -> np.ndarray:
    if hasattr(x, "detach"):             # a torch CPU tensor
        x = x.detach().to("cpu").float().numpy()
    return np.asarray(x, dtype=np.float64)


def attention_bwd(q, k, v, do, scale: float, causal: bool, row_band: int = 2048):
    """Return (dQ, dK, dV) in float64 for q, k, v, do of shape [B,H,N,d]
    (k, v may have another length Nk; causal is top-left aligned, key j
    visible to query i iff j <= i)."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    qi = np.arange(Nq)
    kj = np.arange(Nk)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(B):
        for h in range(H):
            for r0 in range(0, Nq, row_band):
                r1 = min(Nq, r0 + row_band)
                s = scale * (q[b, h, r0:r1] @ k[b, h].T)
                if causal:
                    s = np.where(kj[None, :] > qi[r0:r1, None], -np.inf, s)
                e = np.exp(s - s.max(axis=1, keepdims=True))
                p = e / e.sum(axis=1, keepdims=True)                     # softmax rows
                g = do[b, h, r0:r1]
                dv[b, h] += p.T @ g
                dp = g @ v[b, h].T
                ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
                dq[b, h, r0:r1] = scale * (ds @ k[b, h])
                dk[b, h] += scale * (ds.T @ q[b, h, r0:r1])
    return dq, dk, dv
