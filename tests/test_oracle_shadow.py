"""Pins for the oracle's learner-side shadow-mask attention (CPU only).

Shadow Mask Distillation page, section 1 and Figure 1 caption: the learner
replays the rollout's recorded keep masks in its causal attention, which
makes its policy the rollout's sparse policy. Pinned by: the all-ones mask
against ``torch.nn.functional.scaled_dot_product_attention`` (causal, float64);
that time-frozen alignment itself, against the decode-path oracle on K/V that
both encodings represent exactly; a row that keeps only its own position; and
prompt rows, which ignore the record.
"""
import math

import numpy as np
import pytest
import torch

from oracle import policy, reference, regions, shadow


def rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


@pytest.mark.parametrize("T,Hq,Hkv,P", [(40, 4, 1, 0), (64, 8, 2, 17), (33, 4, 4, 33)])
def test_all_ones_is_causal_attention(T, Hq, Hkv, P):
    D = 32
    q, k, v = rand((T, Hq, D), 1), rand((T, Hkv, D), 2), rand((T, Hkv, D), 3)
    rows = np.ones((T - P, Hkv, T), bool)
    out, lse = shadow.shadow_attention(q, k, v, P, rows)
    G = Hq // Hkv
    qt = torch.from_numpy(q).permute(1, 0, 2)[None]
    kt = torch.from_numpy(np.repeat(k, G, axis=1)).permute(1, 0, 2)[None]
    vt = torch.from_numpy(np.repeat(v, G, axis=1)).permute(1, 0, 2)[None]
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True)[0]
    np.testing.assert_allclose(out, ref.permute(1, 0, 2).numpy(), rtol=1e-12, atol=1e-12)
    # lse from its definition
    s = np.einsum("thd,jhd->thj", q, np.repeat(k, G, axis=1)) / math.sqrt(D)
    s = np.where(np.tril(np.ones((T, T), bool))[:, None, :], s, -np.inf)
    mx = s.max(axis=2, keepdims=True)
    ref_lse = mx[..., 0] + np.log(np.exp(s - mx).sum(axis=2))
    np.testing.assert_allclose(lse, ref_lse, rtol=1e-12)


def doubly_exact_rows(L, D, seed):
    """Integer rows that INT4 (per group of 32: 16 consecutive integers with both
    ends present) and INT8 (max |x| = 127, so s = 1) both represent exactly."""
    rng = np.random.default_rng(seed)
    x = np.empty((L, D), np.float32)
    for t in range(L):
        for g in range(D // 32):
            lo = int(rng.integers(-127, 113))
            codes = rng.integers(0, 16, 32)
            codes[0], codes[1] = 0, 15
            x[t, g * 32:(g + 1) * 32] = lo + codes
        g = int(rng.integers(0, D // 32))
        x[t, g * 32:(g + 1) * 32] = x[t, g * 32:(g + 1) * 32] - x[t, g * 32:(g + 1) * 32].min() + 112
    return x


@pytest.mark.parametrize("budget", [0, 300, 1000])
def test_time_frozen_alignment_with_the_decode_path(budget):
    """With shadow row p = the keep mask of the decode step at length p + 1, the
    learner's row p is the rollout's decode attention at that step."""
    T, P, D, Hkv, G = 420, 150, 64, 2, 2
    k = np.stack([doubly_exact_rows(T, D, 10 + g) for g in range(Hkv)], axis=1)
    v = np.stack([doubly_exact_rows(T, D, 20 + g) for g in range(Hkv)], axis=1)
    for x in (k, v):  # both encodings are exact on these rows
        enc = reference.encode(x[:, 0], x[:, 0])
        kh, _ = reference.decoded(enc)
        assert np.array_equal(kh, x[:, 0].astype(np.float64))
    q = rand((T, Hkv * G, D), 4) * 0.02
    scores = rand((Hkv, T), 5)
    rows = np.zeros((T - P, Hkv, T), bool)
    keeps = {}
    for p in range(P, T):
        L = p + 1
        start, n4 = regions.int4_range(L)
        for g in range(Hkv):
            keep4 = policy.topk_keep(scores[g, start:start + n4], budget)
            keeps[p, g] = keep4
            rows[p - P, g, regions.int8_positions(L)] = True
            rows[p - P, g, start + np.nonzero(keep4)[0]] = True
    out, lse = shadow.shadow_attention(q, k, v, P, rows)
    for p in range(P, T):
        for g in range(Hkv):
            hs = slice(g * G, (g + 1) * G)
            ro, rl = reference.decode_group(q[p, hs], k[: p + 1, g], v[: p + 1, g], keeps[p, g])
            np.testing.assert_allclose(out[p, hs], ro, rtol=1e-11, atol=1e-10)
            np.testing.assert_allclose(lse[p, hs], rl, rtol=1e-12)


def test_row_keeping_only_itself():
    T, P, D = 30, 5, 16
    q, k, v = rand((T, 2, D), 6), rand((T, 1, D), 7), rand((T, 1, D), 8)
    rows = np.zeros((T - P, 1, T), bool)
    for r in range(T - P):
        rows[r, 0, P + r] = True
        rows[r, 0, P + r + 1:] = True  # above the diagonal: ignored
    out, lse = shadow.shadow_attention(q, k, v, P, rows)
    for p in range(P, T):
        np.testing.assert_array_equal(out[p], np.repeat(v[p], 2, axis=0))
        np.testing.assert_allclose(lse[p], q[p] @ k[p, 0] / math.sqrt(D), rtol=1e-14)


def test_prompt_rows_ignore_the_record_and_empty_rows_attend_nothing():
    T, P, D = 24, 10, 16
    q, k, v = rand((T, 2, D), 9), rand((T, 2, D), 10), rand((T, 2, D), 11)
    rows = np.zeros((T - P, 2, T), bool)
    out, lse = shadow.shadow_attention(q, k, v, P, rows)
    dense, dlse = shadow.shadow_attention(q, k, v, T, rows[:0])
    np.testing.assert_array_equal(out[:P], dense[:P])
    np.testing.assert_array_equal(lse[:P], dlse[:P])
    assert np.all(out[P:] == 0.0) and np.all(np.isneginf(lse[P:]))
