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

Block policy (KVP promo page, section "Engineering limits": a paged cache
evicts whole blocks, so token scores are averaged per block before ranking,
and a coarse recency cut to the most recent positions comes before the
learned selection). Readings: block j of B tokens covers the INT4-region
offsets [Bj, Bj+B), offset = position - 16, so with B = 16 the blocks are
whole pages (the section names 16, 32 and 64 as sizes to try);
the candidates are the INT4-region positions, or with a window W > 0 only
the last W of them; a block's score is the float32 mean of its candidate
positions' scores (summed in position order, then divided by their count);
k = floor(budget_permille * nb / 1000) of the nb candidate blocks are kept,
ordered like tokens (score descending, then block index ascending, NaN
last); every candidate position of a kept block is kept.
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


def block_keep(scores_int4, budget_permille: int, block: int = 16, window: int = 0):
    """Keep flags (bool [n4]) under the block policy for INT4-region scores given in
    position order from position 16 (a block boundary)."""
    s = np.asarray(scores_int4, np.float32)
    n4 = s.shape[0]
    keep = np.zeros(n4, dtype=bool)
    c0 = max(0, n4 - window) if window > 0 else 0  # first candidate (region offset)
    if n4 == 0 or c0 >= n4:
        return keep
    j0 = c0 // block
    j1 = (n4 + block - 1) // block
    means = np.zeros(j1 - j0, dtype=np.float32)
    for j in range(j0, j1):
        a, b = max(block * j, c0), min(block * j + block, n4)
        acc = np.float32(0.0)
        for t in range(a, b):          # position order, float32
            acc = np.float32(acc + s[t])
        means[j - j0] = np.float32(acc / np.float32(b - a))
    nb = j1 - j0
    k = (int(budget_permille) * nb) // 1000
    m = means.astype(np.float64)
    nan = np.isnan(m)
    m[nan] = -np.inf
    idx = np.arange(nb)
    order = np.lexsort((idx, -m, nan))
    for jj in order[:k]:
        j = j0 + int(jj)
        keep[max(block * j, c0):min(block * j + block, n4)] = True
    return keep
