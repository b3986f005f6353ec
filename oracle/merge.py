"""Merging partial attentions through their log-sum-exps, in float64.

TEST INFRASTRUCTURE ONLY (see the package docstring): imported by the tests,
never by the product path, and sharing no code with it.

The online softmax of the "Flash Attention" glossary page (second paragraph)
accumulates partial results key block by key block; the same page (fourth
paragraph) names ring attention, which spreads that tiling over devices and
long-context inference.  Both rest on one identity of the softmax definition:
if the keys of a row are split into disjoint parts s with partial results
O_s = sum_{j in s} exp(S_j - LSE_s) V_j and LSE_s = ln sum_{j in s} exp(S_j),
then over all keys

    LSE = ln sum_s exp(LSE_s),        O = sum_s exp(LSE_s - LSE) O_s.

A part with no visible key has LSE_s = -inf and weight exp(-inf) = 0, whatever
its O_s (taken as 0).
"""
from __future__ import annotations

import numpy as np


def lse_merge(o_parts, lse_parts):
    """o_parts [P, ..., d], lse_parts [P, ...] -> (O [..., d], LSE [...]) in float64.

    Rows whose parts are all -inf get O = 0 and LSE = -inf."""
    o_parts = np.asarray(o_parts, dtype=np.float64)
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    m = lse_parts.max(axis=0)                                   # largest part per row
    m_safe = np.where(np.isfinite(m), m, 0.0)
    w = np.where(np.isfinite(lse_parts), np.exp(lse_parts - m_safe), 0.0)   # exp(LSE_s - m)
    den = w.sum(axis=0)
    lse = np.where(den > 0, m_safe + np.log(np.where(den > 0, den, 1.0)), -np.inf)
    num = (w[..., None] * np.where(np.isfinite(lse_parts)[..., None], o_parts, 0.0)).sum(axis=0)
    o = np.where((den > 0)[..., None], num / np.where(den > 0, den, 1.0)[..., None], 0.0)
    return o, lse


def decode_positions(n_q: int, n_k: int) -> np.ndarray:
    """Sequence positions of n_q queries that are the last n_q of n_k tokens
    (causal attention of a decode step: query i sees keys 0 .. n_k - n_q + i)."""
    return np.arange(n_k - n_q, n_k, dtype=np.int64)
