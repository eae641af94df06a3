"""Pins for the dense bfloat16 baseline oracle (CPU only).

The KV4-RL review (section 3) measures the INT4 cache against BF16 rollout,
whose cache holds every K/V row in bfloat16 and attends to every position.
These tests pin ``oracle.dense`` by: bfloat16 rounding against torch's own
float32 -> bfloat16 conversion and against hand cases that follow from the
format (ties to even, carry into the exponent, overflow); the composition
against the compressed-cache oracle on rows that INT4 and bfloat16 both hold
exactly (pure KV4 with nothing evicted reads the same values); L = 1 (the
output is the single value row); and brute force with ``math.fsum`` over
values stored through torch's conversion.
"""
import math

import numpy as np
import pytest
import torch

from oracle import dense, reference


def f32_from_bits(b):
    return np.array(b, dtype=np.uint32).view(np.float32)


@pytest.mark.parametrize("seed", range(3))
def test_bf16_round_matches_torch_conversion(seed):
    rng = np.random.default_rng(seed)
    bits = rng.integers(0, 2**32, 200_000, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    x = x[~np.isnan(x)]
    ours = dense.bf16_round(x)
    ref = torch.from_numpy(x.copy()).to(torch.bfloat16).to(torch.float32).numpy()
    np.testing.assert_array_equal(ours.view(np.uint32), ref.view(np.uint32))


def test_bf16_round_hand_cases():
    one = 0x3F800000
    cases = [
        (one, one),                      # exact
        (one + 0x8000, one),             # 1 + 2^-8: halfway, kept part even -> down
        (one + 0x18000, one + 0x20000),  # 1 + 3*2^-8: halfway, kept part odd -> up to 1 + 2^-6
        (one + 0x8001, one + 0x10000),   # just above halfway -> up
        (one + 0x7FFF, one),             # just below halfway -> down
        (0xBF808000, 0xBF800000),        # -(1 + 2^-8) -> -1
        (0x3FFFFFFF, 0x40000000),        # carry into the exponent: just below 2 -> 2
        (0x7F7F7FFF, 0x7F7F0000),        # largest bfloat16 stays
        (0x7F7F8000, 0x7F800000),        # halfway above the largest bfloat16 -> inf
        (0x7F800000, 0x7F800000),        # inf
        (0x00000001, 0x00000000),        # smallest subnormal -> 0
        (0x00008000, 0x00000000),        # halfway between 0 and the smallest bf16 subnormal -> even (0)
        (0x00018000, 0x00020000),        # halfway, odd -> up
    ]
    x = f32_from_bits([c[0] for c in cases])
    got = dense.bf16_round(x).view(np.uint32)
    assert [hex(g) for g in got] == [hex(c[1]) for c in cases]
    assert np.isnan(dense.bf16_round(np.float32(np.nan)))


def test_bf16_rows_are_stored_unchanged():
    x = dense.bf16_round(np.random.default_rng(5).standard_normal((7, 64)).astype(np.float32))
    np.testing.assert_array_equal(dense.store_rows(x, "bf16"), x)
    np.testing.assert_array_equal(dense.store_rows(x, "f32"), x)


def exact_rows(L, D, seed):
    """Rows INT4 (group 32, codes 0..15 plus an integer offset) and bfloat16 both hold exactly."""
    rng = np.random.default_rng(seed)
    x = np.empty((L, D), np.float32)
    for t in range(L):
        for g in range(D // 32):
            codes = rng.integers(0, 16, 32)
            codes[0], codes[1] = 0, 15
            x[t, g * 32:(g + 1) * 32] = codes + rng.integers(-20, 20)
    return x


@pytest.mark.parametrize("L", [1, 37, 300])
def test_dense_equals_pure_kv4_with_nothing_evicted_on_exact_rows(L):
    D, G = 64, 4
    k, v = exact_rows(L, D, 31), exact_rows(L, D, 32)
    q = np.random.default_rng(33).standard_normal((G, D)) * 0.05
    out, lse = dense.decode_group(q, k, v, "f32")
    ref_out, ref_lse = reference.decode_group(q, k, v, np.ones(L, bool), n_sink=0, n_recent=0)
    np.testing.assert_allclose(out, ref_out, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse, ref_lse, rtol=1e-13)


def test_single_position_returns_its_value_row():
    D = 128
    rng = np.random.default_rng(40)
    k = rng.standard_normal((1, D)).astype(np.float32)
    v = rng.standard_normal((1, D)).astype(np.float32)
    q = rng.standard_normal((2, D))
    out, lse = dense.decode_group(q, k, v, "f32")
    vb = torch.from_numpy(v[0].copy()).to(torch.bfloat16).double().numpy()
    kb = torch.from_numpy(k[0].copy()).to(torch.bfloat16).double().numpy()
    np.testing.assert_array_equal(out, np.stack([vb, vb]))
    np.testing.assert_allclose(lse, q @ kb / math.sqrt(D), rtol=1e-13)


def test_empty_sequence():
    out, lse = dense.decode_group(np.ones((2, 64)), np.zeros((0, 64)), np.zeros((0, 64)))
    assert (out == 0).all() and np.isneginf(lse).all()


@pytest.mark.parametrize("L", [2, 5])
def test_brute_force_with_torch_storage(L):
    D, G = 64, 2
    rng = np.random.default_rng(50 + L)
    k = (rng.standard_normal((L, D)) * 2).astype(np.float32)
    v = rng.standard_normal((L, D)).astype(np.float32)
    q = rng.standard_normal((G, D))
    out, lse = dense.decode_group(q, k, v, "f32", scale=0.3)
    kb = torch.from_numpy(k).to(torch.bfloat16).double().numpy().tolist()
    vb = torch.from_numpy(v).to(torch.bfloat16).double().numpy().tolist()
    for h in range(G):
        s = [0.3 * math.fsum(q[h][d] * kb[t][d] for d in range(D)) for t in range(L)]
        m = max(s)
        e = [math.exp(x - m) for x in s]
        den = math.fsum(e)
        for d in range(D):
            assert abs(out[h][d] - math.fsum(e[t] * vb[t][d] for t in range(L)) / den) < 1e-12
        assert abs(lse[h] - (m + math.log(den))) < 1e-12
