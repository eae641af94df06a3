"""Composition for one (sequence, kv head): encode, decode, keep set, attend.

Test infrastructure only. Follows the KV4-RL review, section 3 (INT4 for the
full context, INT8 for the 16 sink and 128 recent positions, independent
regions joined by an exact softmax merge) and the Shadow Mask Distillation
page, Figure 1 caption (a binary mask of retained indices). Since the merge is
exact, the result is attention over the union of the INT8 positions and the
kept INT4 positions, each read through its own encoding.

``n_sink = n_recent = 0`` is the unprotected configuration the same section
compares against ("pure KV4"): no INT8 positions, every position read from
INT4 and subject to the keep mask.
"""
from __future__ import annotations

import numpy as np

from . import attention, policy, quant, regions


def encode(k_src, v_src, n_sink=regions.N_SINK, n_recent=regions.N_RECENT):
    """Encode a sequence's source K and V (float32 [L][D]).

    INT4 codes are produced for every position; INT8 codes only for the
    protected positions (returned in the order of ``regions.int8_positions``).
    """
    k_src = np.asarray(k_src, np.float32)
    v_src = np.asarray(v_src, np.float32)
    L = k_src.shape[0]
    k4, ks4, km4 = quant.int4_encode(k_src)
    v4, vs4, vm4 = quant.int4_encode(v_src)
    pos8 = regions.int8_positions(L, n_sink, n_recent)
    k8, ks8 = quant.int8_encode(k_src[pos8])
    v8, vs8 = quant.int8_encode(v_src[pos8])
    return {
        "L": L, "pos8": pos8, "n_sink": n_sink, "n_recent": n_recent,
        "k4": k4, "k4_scale": ks4, "k4_min": km4,
        "v4": v4, "v4_scale": vs4, "v4_min": vm4,
        "k8": k8, "k8_scale": ks8, "v8": v8, "v8_scale": vs8,
    }


def decoded(enc):
    """Float64 K-hat, V-hat [L][D]: INT8 decoding on protected positions, INT4 elsewhere."""
    k = quant.int4_decode(enc["k4"], enc["k4_scale"], enc["k4_min"])
    v = quant.int4_decode(enc["v4"], enc["v4_scale"], enc["v4_min"])
    pos8 = enc["pos8"]
    if pos8.shape[0]:
        k[pos8] = quant.int8_decode(enc["k8"], enc["k8_scale"])
        v[pos8] = quant.int8_decode(enc["v8"], enc["v8_scale"])
    return k, v


def kept_positions(L: int, keep4, n_sink=regions.N_SINK, n_recent=regions.N_RECENT) -> np.ndarray:
    """Sorted attended positions: INT8 positions plus the kept INT4-region positions."""
    start, n4 = regions.int4_range(L, n_sink, n_recent)
    keep4 = np.asarray(keep4, bool)
    if keep4.shape[0] != n4:
        raise ValueError(f"keep4 has {keep4.shape[0]} flags, INT4 region has {n4}")
    kept4 = start + np.nonzero(keep4)[0]
    return np.sort(np.concatenate([regions.int8_positions(L, n_sink, n_recent), kept4]))


def decode_group(q, k_src, v_src, keep4, scale=None, n_sink=regions.N_SINK,
                 n_recent=regions.N_RECENT):
    """Output (float64 [G][D]) and LSE ([G]) for the G query heads of one kv head."""
    enc = encode(k_src, v_src, n_sink, n_recent)
    k_hat, v_hat = decoded(enc)
    pos = kept_positions(enc["L"], keep4, n_sink, n_recent)
    return attention.attend(q, k_hat[pos], v_hat[pos], scale)


def keep_from_scores(scores, L: int, budget_permille: int, n_sink=regions.N_SINK,
                     n_recent=regions.N_RECENT):
    """Top-k keep flags of the INT4 region from per-position scores ([>= L])."""
    start, n4 = regions.int4_range(L, n_sink, n_recent)
    return policy.topk_keep(np.asarray(scores)[start:start + n4], budget_permille)
