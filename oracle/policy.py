"""Per-head scoring MLP and budgeted top-k keep set (oracle; test infrastructure only).

Sources: the KVP promo page for arXiv 2602.10238, section "Core mechanism":
one small MLP per attention head whose input is the K/V vectors themselves
and whose output is one utility score per token; deployment is score, sort,
truncate to the budget (any budget from 10% to 90%). The TTKV promo page
(arXiv 2604.19769), first insight: eviction as ranking with a continuous score.
The Shadow Mask Distillation page (arXiv 2605.06850), Figure 1 caption: the
eviction records the retained indices into a binary mask M.

Readings: the MLP is 2D -> 32 -> ReLU -> 1 on the source K||V (float32
widened to float64 here); no output squashing (monotone, so top-k is
unchanged). The budget applies per (sequence, kv head) to the INT4 region:
k = floor(budget_permille * n4 / 1000); order by score descending, then
position ascending; NaN ranks below every number, -inf included (so the
order is total and the kept set unique).
"""
from __future__ import annotations

import numpy as np

HIDDEN = 32


def unpack_mlp(w, head_dim: int):
    """Split one head's flat weights [8257 at D=128] into (W1 [32][2D], b1 [32], w2 [32], b2)."""
    w = np.asarray(w, np.float64)
    d2 = 2 * head_dim
    n1 = HIDDEN * d2
    W1 = w[:n1].reshape(HIDDEN, d2)
    b1 = w[n1:n1 + HIDDEN]
    w2 = w[n1 + HIDDEN:n1 + 2 * HIDDEN]
    b2 = w[n1 + 2 * HIDDEN]
    return W1, b1, w2, b2


def mlp_scores(k, v, w):
    """Scores w2 . relu(W1 [k || v] + b1) + b2 for rows of k, v (float [N][D]); float64 [N]."""
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    W1, b1, w2, b2 = unpack_mlp(w, k.shape[-1])
    x = np.concatenate([k, v], axis=-1)
    h = np.maximum(x @ W1.T + b1, 0.0)
    return h @ w2 + b2


def budget_k(n4: int, budget_permille: int) -> int:
    """Number of INT4-region positions kept: floor(budget_permille * n4 / 1000)."""
    return (int(budget_permille) * int(n4)) // 1000


def topk_keep(scores_int4, budget_permille: int):
    """Keep flags (bool [n4]) for the INT4-region scores given in position order."""
    s = np.asarray(scores_int4, np.float64).copy()
    n4 = s.shape[0]
    k = budget_k(n4, budget_permille)
    nan = np.isnan(s)
    s[nan] = -np.inf
    pos = np.arange(n4)
    # primary: numbers before NaN; then score descending; then position ascending
    order = np.lexsort((pos, -s, nan))
    keep = np.zeros(n4, dtype=bool)
    keep[order[:k]] = True
    return keep
