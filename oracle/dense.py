"""Dense bfloat16 paged-KV decode attention (oracle; test infrastructure only).

Source: KV4-RL review, section 3 "Method & Key Results": the rollout speedups
of the INT4 cache are measured against BF16 rollout, i.e. decoding over a KV
cache that stores every K and V row in bfloat16 and attends to every cached
position. This module is that baseline's attention for one (sequence, kv
head): no quantization, no keep mask, no protected region.

Readings (the pages fix none of these): a float32 source row is stored as its
bfloat16 round-to-nearest-even (a bfloat16 source row is stored unchanged);
the query is used as given (bfloat16 queries widened exactly); logits are
(q . k) * scale with scale = 1/sqrt(D) unless given; positions [0, L) are all
attended, L = 0 gives output 0 and LSE = -inf. Attention itself is the plain
definition of :func:`oracle.attention.attend` in float64.
"""
from __future__ import annotations

import numpy as np

from . import attention


def bf16_round(x) -> np.ndarray:
    """float32 values rounded to the nearest bfloat16 (ties to even), as float32.

    bfloat16 keeps the top 16 bits of an IEEE binary32 value (sign, 8 exponent
    bits, 7 mantissa bits). Rounding to nearest-even adds half of the dropped
    unit, minus one when the kept part is even, before truncating; overflow
    carries into the exponent (up to infinity). NaN stays NaN (quiet).
    """
    x = np.ascontiguousarray(np.asarray(x, np.float32))
    u = x.view(np.uint32).astype(np.uint64)
    keep_lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + keep_lsb) >> np.uint64(16)) << np.uint64(16)
    out = (r & np.uint64(0xFFFFFFFF)).astype(np.uint32).view(np.float32)
    return np.where(np.isnan(x), np.float32(np.nan), out).astype(np.float32)


def store_rows(rows, src_dtype: str) -> np.ndarray:
    """Values the dense cache holds for source rows: bfloat16 rows as they are,
    float32 rows rounded to bfloat16 (float32 array either way)."""
    rows = np.asarray(rows, np.float32)
    return rows if src_dtype == "bf16" else bf16_round(rows)


def decode_group(q, k_rows, v_rows, src_dtype: str = "f32", scale=None):
    """Output (float64 [G][D]) and LSE ([G]) of the G query heads of one kv head
    over every position of a dense bfloat16 cache built from source rows
    ``k_rows``, ``v_rows`` (float32 values [L][D])."""
    k = store_rows(k_rows, src_dtype)
    v = store_rows(v_rows, src_dtype)
    return attention.attend(q, k, v, scale)
