"""Masked softmax attention for one decode query group (oracle; test infrastructure only).

Source: KV4-RL review, section 3: the INT4 region and the protected INT8
region are processed independently and their outputs combined by an exact
softmax merge, without reconstructing the full cache. Reaching exactly the
plain result is the point of that merge, so :func:`attend` computes the plain
definition over the union of kept positions in float64; :func:`partial` and
:func:`merge` exist only for the invariant tests that check the merge.

Readings: logits are (q . k) / sqrt(D) unless a scale is given; query head h
uses kv head floor(h / G); an empty key set gives LSE = -inf and output 0.
"""
from __future__ import annotations

import numpy as np


def attend(q, keys, values, scale=None):
    """Softmax attention of queries q [G][D] over keys/values [N][D], float64.

    Returns (out [G][D], lse [G]); lse is the natural-log log-sum-exp of the
    scaled logits.
    """
    q = np.asarray(q, np.float64)
    keys = np.asarray(keys, np.float64)
    values = np.asarray(values, np.float64)
    G, D = q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    if keys.shape[0] == 0:
        return np.zeros((G, values.shape[-1] if values.ndim == 2 else D)), np.full(G, -np.inf)
    s = (q @ keys.T) * scale
    m = s.max(axis=1)
    p = np.exp(s - m[:, None])
    l = p.sum(axis=1)
    out = (p @ values) / l[:, None]
    return out, m + np.log(l)


def partial(q, keys, values, scale=None):
    """Unnormalised partial (m, l, o) over one subset of keys; empty -> (-inf, 0, 0)."""
    q = np.asarray(q, np.float64)
    G, D = q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    keys = np.asarray(keys, np.float64)
    values = np.asarray(values, np.float64)
    if keys.shape[0] == 0:
        return np.full(G, -np.inf), np.zeros(G), np.zeros((G, values.shape[-1]))
    s = (q @ keys.T) * scale
    m = s.max(axis=1)
    p = np.exp(s - m[:, None])
    return m, p.sum(axis=1), p @ values


def merge(parts):
    """Exact log-sum-exp merge of partials [(m, l, o), ...] -> (out, lse).

    M = max_j m_j; w_j = exp(m_j - M) (0 for empty partials);
    out = sum_j w_j o_j / sum_j w_j l_j; lse = M + ln(sum_j w_j l_j).
    """
    ms = np.stack([p[0] for p in parts])
    M = ms.max(axis=0)
    G = M.shape[0]
    finite = np.isfinite(M)
    Ms = np.where(finite, M, 0.0)
    num = np.zeros_like(parts[0][2])
    den = np.zeros(G)
    for m, l, o in parts:
        w = np.where(np.isfinite(m), np.exp(np.where(np.isfinite(m), m, 0.0) - Ms), 0.0)
        num = num + w[:, None] * o
        den = den + w * l
    out = np.where(den[:, None] > 0, num / np.where(den > 0, den, 1.0)[:, None], 0.0)
    lse = np.where(den > 0, Ms + np.log(np.where(den > 0, den, 1.0)), -np.inf)
    return out, lse
