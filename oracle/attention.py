"""Plain fp64 attention: the definition the fused kernels must reproduce.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and
the benchmark's CPU-baseline leg may import this module; the product path
never calls it.  It shares no code with the GPU path.

What is computed (the pages' "standard attention", which materialises the
whole N x N score matrix; FlashAttention is said to return numerically the
same result, only computed tile by tile):
  - "Flash Attention" glossary page (news.hamidun.com), first and second
    paragraphs: standard attention materialises the full N x N matrix in HBM,
    FlashAttention gives the same result and never writes that matrix;
  - "FlashAttention-3 (PT)", section "O problema do mecanismo de atencao": the
    softmax over the attention matrix and its O(n^2) intermediate tensor.

Readings where the pages are silent (the causal mask, the LSE output and the
layout are not on the pages):
  - layout [B, H, N, d], contiguous rows;
  - causal means square, top-left aligned: key j is visible to query i iff
    j <= i (query index taken from ``q_index`` when only some rows are asked);
  - LSE_i = m_i + ln(l_i), the natural log of the sum of exp over the scaled,
    masked scores of row i.

Per (b, h), in float64:
  S = scale * Q K^T; S_ij = -inf where masked; m_i = max_j S_ij;
  P_ij = exp(S_ij - m_i); l_i = sum_j P_ij; O_i = (sum_j P_ij V_j) / l_i;
  LSE_i = m_i + ln l_i.
Full rows of S are always formed; long sequences are processed a band of
complete rows at a time, which does not change any row's arithmetic.
"""
from __future__ import annotations

import numpy as np


def _f64(x) -> np.ndarray:
    if hasattr(x, "detach"):             # a torch CPU tensor
        x = x.detach().to("cpu").float().numpy()
    return np.asarray(x, dtype=np.float64)


def attention(q, k, v, scale: float, causal: bool, q_index=None, row_band: int = 4096):
    """Return (O, LSE) in float64 for q [B,H,Nq,d], k [B,H,Nk,d], v [B,H,Nk,dv].

    ``q_index`` (length Nq) gives each query row's position in the sequence for
    the causal mask; by default rows are positions 0..Nq-1.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    dv = v.shape[3]
    qi = np.arange(Nq) if q_index is None else np.asarray(q_index, dtype=np.int64)
    kj = np.arange(Nk)
    o = np.empty((B, H, Nq, dv), dtype=np.float64)
    lse = np.empty((B, H, Nq), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            for r0 in range(0, Nq, row_band):
                r1 = min(Nq, r0 + row_band)
                s = scale * (q[b, h, r0:r1] @ k[b, h].T)               # rows r0..r1 of S
                if causal:
                    s = np.where(kj[None, :] > qi[r0:r1, None], -np.inf, s)
                m = s.max(axis=1, keepdims=True)
                p = np.exp(s - m)
                l = p.sum(axis=1, keepdims=True)
                o[b, h, r0:r1] = (p @ v[b, h]) / l
                lse[b, h, r0:r1] = (m + np.log(l))[:, 0]
    return o, lse

