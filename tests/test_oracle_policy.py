"""Pins for the oracle's scoring MLP and top-k keep set (CPU only).

KVP promo page (arXiv 2602.10238), "Core mechanism": one small MLP per head
over the K/V vectors gives each token a score; deployment ranks by score and
truncates to the budget. The oracle is pinned against a naive Python
evaluation of the MLP, against a full Python sort of (score desc, position
asc), and against the invariants every top-k must satisfy.
"""
import math

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

from golden.read import constants
from oracle import policy


def naive_mlp(k, v, w, D):
    x = list(k) + list(v)
    n1 = 32 * 2 * D
    h = []
    for j in range(32):
        a = math.fsum(w[j * 2 * D + i] * x[i] for i in range(2 * D)) + w[n1 + j]
        h.append(max(a, 0.0))
    return math.fsum(w[n1 + 32 + j] * h[j] for j in range(32)) + w[n1 + 64]


@pytest.mark.parametrize("D", [64, 128])
def test_mlp_matches_naive_loops(D):
    rng = np.random.default_rng(D)
    w = rng.standard_normal(32 * 2 * D + 65) * 0.1
    k = rng.standard_normal((5, D))
    v = rng.standard_normal((5, D))
    got = policy.mlp_scores(k, v, w)
    for i in range(5):
        assert abs(got[i] - naive_mlp(k[i], v[i], w.tolist(), D)) < 1e-12


def test_mlp_relu_and_bias_terms():
    D = 64
    w = np.zeros(32 * 2 * D + 65)
    w[-1] = 2.5                      # b2 only
    assert policy.mlp_scores(np.ones((1, D)), np.ones((1, D)), w)[0] == 2.5
    w[32 * 2 * D] = -1.0             # b1[0] negative: ReLU clips it
    w[32 * 2 * D + 32] = 7.0         # w2[0]
    assert policy.mlp_scores(np.zeros((1, D)), np.zeros((1, D)), w)[0] == 2.5
    w[32 * 2 * D] = 1.0
    assert policy.mlp_scores(np.zeros((1, D)), np.zeros((1, D)), w)[0] == 9.5


def test_mlp_size_is_the_pages_8k():
    c = constants()
    n = 32 * 2 * 128 + 32 + 32 + 1
    assert n == 8257 and abs(n - c["mlp_params_approx"][0]) < 300


def python_topk(scores, budget):
    n = len(scores)
    k = budget * n // 1000
    key = [(1, 0.0, i) if s != s else (0, -s, i) for i, s in enumerate(scores)]
    chosen = sorted(range(n), key=lambda i: key[i])[:k]
    out = [False] * n
    for i in chosen:
        out[i] = True
    return out


@settings(max_examples=300, deadline=None)
@given(st.lists(st.one_of(st.floats(allow_nan=True, allow_infinity=True, width=32),
                          st.sampled_from([0.0, 1.0, -1.0])), max_size=200),
       st.integers(0, 1000))
def test_topk_matches_full_python_sort(scores, budget):
    got = policy.topk_keep(np.array(scores, np.float32), budget)
    assert got.tolist() == python_topk(scores, budget)


def test_topk_invariants():
    rng = np.random.default_rng(0)
    s = rng.standard_normal(5000)
    for budget in (100, 300, 500, 900, 1000, 0):
        keep = policy.topk_keep(s, budget)
        k = budget * 5000 // 1000
        assert keep.sum() == k
        if 0 < k < 5000:
            assert s[keep].min() >= s[~keep].max()


def test_topk_ties_keep_lower_positions():
    s = np.array([1.0, 2.0, 1.0, 1.0, 2.0, 1.0])
    assert policy.topk_keep(s, 500).tolist() == [True, True, False, False, True, False]


def test_topk_nan_ranks_last():
    s = np.array([np.nan, -1e30, np.nan, -np.inf])
    assert policy.topk_keep(s, 500).tolist() == [False, True, False, True]
    assert policy.topk_keep(s, 750).tolist() == [True, True, False, True]


def test_budget_k_floor():
    assert policy.budget_k(130928, 100) == 13092
    assert policy.budget_k(130928, 500) == 65464
    assert policy.budget_k(32624, 300) == 9787
    assert policy.budget_k(7, 1000) == 7 and policy.budget_k(7, 0) == 0
    c = constants()
    assert c["budget_min_percent"][0] == 10 and c["budget_max_percent"][0] == 90


# ------------------------------------------------------------- block policy
def fraction_block_keep(scores, budget, block, window):
    """Independent pin: exact rational block means, Python sort."""
    from fractions import Fraction

    n4 = len(scores)
    c0 = max(0, n4 - window) if window > 0 else 0
    keep = [False] * n4
    if c0 >= n4:
        return np.array(keep)
    blocks = []
    j = c0 // block
    while block * j < n4:
        a, b = max(block * j, c0), min(block * j + block, n4)
        mean = Fraction(sum(int(x) for x in scores[a:b]), b - a)
        blocks.append((-mean, j, a, b))
        j += 1
    k = budget * len(blocks) // 1000
    for _, _, a, b in sorted(blocks)[:k]:
        for t in range(a, b):
            keep[t] = True
    return np.array(keep)


@settings(max_examples=300, deadline=None)
@given(st.lists(st.integers(-50, 50), min_size=0, max_size=200), st.integers(0, 1000),
       st.sampled_from([0, 1, 7, 16, 33, 100, 1000]))
def test_block_policy_matches_exact_rational_ranking(ints, budget, window):
    # integer scores: float32 sums are exact and distinct means stay distinct
    scores = np.array(ints, np.float32)
    got = policy.block_keep(scores, budget, 16, window)
    np.testing.assert_array_equal(got, fraction_block_keep(ints, budget, 16, window))


@settings(max_examples=200, deadline=None)
@given(st.lists(st.floats(-1e3, 1e3, width=32), min_size=0, max_size=120), st.integers(0, 1000))
def test_block_policy_with_one_token_blocks_is_token_topk(vals, budget):
    s = np.array(vals, np.float32)
    np.testing.assert_array_equal(policy.block_keep(s, budget, block=1), policy.topk_keep(s, budget))


def test_block_policy_hand_cases():
    # three full blocks with means 1, 3, 2; 66.7% of 3 blocks -> 2 blocks: the 3s and the 2s
    s = np.repeat(np.array([1.0, 3.0, 2.0], np.float32), 16)
    keep = policy.block_keep(s, 667)
    assert not keep[:16].any() and keep[16:].all()
    # 40 positions scored by index, window 20: candidates 20..39 in blocks
    # [20, 32) (mean 25.5) and [32, 40) (mean 35.5); half of 2 blocks keeps the second
    s = np.arange(40, dtype=np.float32)
    keep = policy.block_keep(s, 500, window=20)
    assert keep[32:].all() and not keep[:32].any()
    # budget 1000 keeps every candidate, none before the window
    keep = policy.block_keep(s, 1000, window=20)
    assert keep[20:].all() and not keep[:20].any()
    # ties keep the lower block; a NaN block ranks below -inf
    s = np.concatenate([np.full(16, 5.0), np.full(16, 5.0), np.full(16, -np.inf), np.full(16, np.nan)]).astype(np.float32)
    assert policy.block_keep(s, 250)[:16].all() and not policy.block_keep(s, 250)[16:].any()
    keep = policy.block_keep(s, 750)
    assert keep[:48].all() and not keep[48:].any()


def test_block_policy_invariants():
    rng = np.random.default_rng(7)
    for _ in range(50):
        n4 = int(rng.integers(0, 400))
        s = rng.standard_normal(n4).astype(np.float32)
        budget = int(rng.integers(0, 1001))
        window = int(rng.choice([0, 10, 64, 200]))
        keep = policy.block_keep(s, budget, 16, window)
        c0 = max(0, n4 - window) if window > 0 else 0
        assert not keep[:c0].any()
        # whole candidate blocks only
        for j in range(c0 // 16, (n4 + 15) // 16):
            a, b = max(16 * j, c0), min(16 * j + 16, n4)
            assert keep[a:b].all() or not keep[a:b].any()
        nb = (n4 + 15) // 16 - c0 // 16 if n4 > c0 else 0
        kept_blocks = sum(1 for j in range(c0 // 16, (n4 + 15) // 16) if keep[max(16 * j, c0)])
        assert kept_blocks == budget * nb // 1000


def test_block_mean_is_float32_in_position_order():
    """Pins the summation the block policy's reading fixes: a block's score is its
    candidates' scores added one by one in position order in float32, then divided
    by their count. Worked by hand (float32 has an ulp of 8 at 1e8, ties to even):

      block 0 = [1e8, 1 x 15]:    1e8 + 1 rounds back to 1e8 every time -> sum 1e8,
                                  mean 6250000.0 (the exact mean is 6250000.9375)
      block 1 = [1e8, 8, 0 x 14]: 1e8 + 8 = 100000008 is exact -> mean 6250000.5

    so keeping one of the two blocks keeps block 1. Summing in float64 would keep
    block 0 (6250000.9375 > 6250000.5), and numpy's pairwise float32 mean gives
    block 0 100000008 / 16 as well (a tie, which keeps the lower block 0): either
    mistake flips the result.
    """
    a = [1e8] + [1.0] * 15
    b = [1e8, 8.0] + [0.0] * 14
    s = np.array(a + b, np.float32)
    keep = policy.block_keep(s, 500, block=16)
    assert not keep[:16].any() and keep[16:].all()
    # the two other summations really do rank the blocks the other way round
    assert np.float64(np.mean(np.array(a, np.float32))) == np.float64(np.mean(np.array(b, np.float32)))
    assert math.fsum(a) / 16 > math.fsum(b) / 16
    # with the blocks swapped the float32 reading still prefers the [1e8, 8, ...] block
    keep = policy.block_keep(np.array(b + a, np.float32), 500, block=16)
    assert keep[:16].all() and not keep[16:].any()
