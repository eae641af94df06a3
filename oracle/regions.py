"""Which cached positions are INT8 and which are INT4 (oracle; test infrastructure only).

Source: KV4-RL review, section 3: the whole context is stored in paged INT4,
while the first 16 positions (attention sinks) and the 128 most recent cached
positions are protected in an INT8 side cache, so the extra work stays bounded
at any context length. Readings: INT4 codes exist for every position, but
attention reads a position from INT8 when it is protected and from INT4
otherwise, so the two regions are disjoint; a context of L <= 144 positions
has an empty INT4 region; the decode query attends to all L cached positions
including the one just appended.
"""
from __future__ import annotations

import numpy as np

N_SINK = 16
N_RECENT = 128


def int8_positions(L: int, n_sink: int = N_SINK, n_recent: int = N_RECENT) -> np.ndarray:
    """Sorted positions held in INT8: [0, min(L, n_sink)) and [max(n_sink, L - n_recent), L)."""
    sink = np.arange(min(L, n_sink))
    recent = np.arange(max(n_sink, L - n_recent), L)
    return np.concatenate([sink, recent]).astype(np.int64)


def int4_range(L: int, n_sink: int = N_SINK, n_recent: int = N_RECENT):
    """(start, n4): the INT4 region is [start, start + n4), n4 = max(0, L - n_sink - n_recent)."""
    return n_sink, max(0, L - n_sink - n_recent)


def ring_slot(t: int, n_sink: int = N_SINK, n_recent: int = N_RECENT) -> int:
    """INT8 side-cache slot of position t: t for sinks, else n_sink + (t - n_sink) mod n_recent."""
    return t if t < n_sink else n_sink + (t - n_sink) % n_recent
