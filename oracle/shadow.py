"""Learner-side attention under the recorded shadow mask (test infrastructure only).

Source: Shadow Mask Distillation page (arXiv 2605.06850), section 1 and the
Figure 1 caption. During the sparse rollout the eviction algorithm records the
indices it retains at every step into a binary mask M; the learner's alignment
track injects M into its causal attention, so that the learner's query at each
generated position attends to exactly the positions the rollout attended when
it produced that step (a time-frozen mask), which makes the learner's policy
the rollout's sparse policy.

Readings taken here:
* The learner's K and V are its own dense values; M only removes positions
  (the page replays eviction, not quantization).
* Query position p < prompt_len attends densely and causally (the rollout's
  prefill was dense).
* Query position p >= prompt_len uses shadow row r = p - prompt_len: the keep
  mask of the decode step whose query was that of position p, i.e. at cache
  length p + 1 (protected positions included); bits above p are ignored.
* Attention itself is the plain scaled softmax of ``attention.attend``.

Nothing here shares code with the HIP path.
"""
from __future__ import annotations

import numpy as np

from . import attention


def allowed_positions(p: int, prompt_len: int, shadow_row) -> np.ndarray:
    """Key positions the query at position p attends to."""
    causal = np.arange(p + 1)
    if p < prompt_len:
        return causal
    row = np.asarray(shadow_row, bool)
    return causal[row[: p + 1]]


def shadow_attention(q, k, v, prompt_len: int, shadow, scale=None):
    """Causal attention of one sequence with shadow rows for its generated positions.

    q: [T][Hq][D]; k, v: [T][Hkv][D]; shadow: bool [T - prompt_len][Hkv][>= T]
    (row r belongs to query position prompt_len + r). Returns out float64
    [T][Hq][D] and lse float64 [T][Hq] (natural log; -inf when nothing is
    attended).
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    T, Hq, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    out = np.zeros((T, Hq, D))
    lse = np.full((T, Hq), -np.inf)
    for p in range(T):
        for g in range(Hkv):
            row = shadow[p - prompt_len, g] if p >= prompt_len else None
            pos = allowed_positions(p, prompt_len, row)
            hs = slice(g * G, (g + 1) * G)
            out[p, hs], lse[p, hs] = attention.attend(q[p, hs], k[pos, g], v[pos, g], scale)
    return out, lse
