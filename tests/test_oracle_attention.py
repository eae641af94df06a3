"""Pins for the oracle's attention, regions and composition (CPU only).

The KV4-RL review (section 3) says the INT4 and INT8 regions are processed
independently and joined by an exact softmax merge. These tests pin the
oracle by: the merge invariant against a single softmax over the union; the
special case with no quantization and nothing evicted against
``torch.nn.functional.scaled_dot_product_attention`` in float64; brute force
with ``math.fsum`` and 50-digit ``mpmath`` exponentials; the sink+recent-only
special case (k = 0, the StreamingLLM window named on the Shadow Mask
Distillation page, section 2); and inputs that both encodings represent
exactly, which makes the whole composition equal plain attention.
"""
import math

import mpmath
import numpy as np
import pytest
import torch

from golden.read import constants
from oracle import attention, quant, reference, regions


def rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


# ------------------------------------------------------------- merge
@pytest.mark.parametrize("seed", range(6))
def test_merge_of_partials_equals_union_softmax(seed):
    rng = np.random.default_rng(seed)
    G, D, N = 4, 32, 97
    q, k, v = rand((G, D), seed), rand((N, D), seed + 100), rand((N, D), seed + 200)
    nparts = rng.integers(2, 5)
    lab = rng.integers(0, nparts, N)
    lab[rng.integers(0, N)] = 0
    parts = [attention.partial(q, k[lab == j], v[lab == j]) for j in range(nparts)]
    parts.append(attention.partial(q, k[:0], v[:0]))  # an empty split
    out, lse = attention.merge(parts)
    ref_out, ref_lse = attention.attend(q, k, v)
    np.testing.assert_allclose(out, ref_out, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, ref_lse, rtol=1e-12)


def test_merge_all_empty_gives_minus_inf():
    q = rand((2, 8), 1)
    e = np.zeros((0, 8))
    out, lse = attention.merge([attention.partial(q, e, e), attention.partial(q, e, e)])
    assert np.isneginf(lse).all() and (out == 0).all()


# ------------------------------------------------------- library special case
@pytest.mark.parametrize("Hq,Hkv", [(8, 2), (4, 4), (4, 1)])
def test_plain_attention_matches_torch_sdpa(Hq, Hkv):
    D, N = 16, 53
    q = rand((Hq, D), 3)
    k = rand((Hkv, N, D), 4)
    v = rand((Hkv, N, D), 5)
    G = Hq // Hkv
    tq = torch.from_numpy(q)[None, :, None, :]
    tk = torch.from_numpy(k).repeat_interleave(G, dim=0)[None]
    tv = torch.from_numpy(v).repeat_interleave(G, dim=0)[None]
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv)[0, :, 0, :].numpy()
    ref_lse = torch.logsumexp((tq @ tk.transpose(-1, -2))[0, :, 0, :] / math.sqrt(D), dim=-1).numpy()
    for h in range(Hkv):
        out, lse = attention.attend(q[h * G:(h + 1) * G], k[h], v[h])
        np.testing.assert_allclose(out, ref[h * G:(h + 1) * G], rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(lse, ref_lse[h * G:(h + 1) * G], rtol=1e-12)


# ------------------------------------------------------------- brute force
def brute_attend(q, k, v):
    mpmath.mp.dps = 50
    D = len(q[0])
    outs, lses = [], []
    for qh in q:
        s = [math.fsum(qh[i] * kt[i] for i in range(D)) / math.sqrt(D) for kt in k]
        m = max(s)
        p = [mpmath.exp(mpmath.mpf(st) - mpmath.mpf(m)) for st in s]
        l = mpmath.fsum(p)
        outs.append([float(mpmath.fsum(p[t] * mpmath.mpf(v[t][d]) for t in range(len(k))) / l)
                     for d in range(len(v[0]))])
        lses.append(float(mpmath.mpf(m) + mpmath.log(l)))
    return np.array(outs), np.array(lses)


@pytest.mark.parametrize("N", [1, 2, 17, 64])
def test_attention_matches_brute_force(N):
    q, k, v = rand((3, 8), N), rand((N, 8), N + 1) * 3, rand((N, 8), N + 2)
    out, lse = attention.attend(q, k, v)
    bo, bl = brute_attend(q.tolist(), k.tolist(), v.tolist())
    np.testing.assert_allclose(out, bo, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(lse, bl, rtol=1e-13, atol=1e-14)


# ------------------------------------------------------------- regions
def test_region_constants_are_the_pages():
    c = constants()
    assert regions.N_SINK == c["n_sink"][0]
    assert regions.N_RECENT == c["n_recent"][0]


def test_regions_hand_examples():
    assert regions.int8_positions(150).tolist() == list(range(16)) + list(range(22, 150))
    assert regions.int4_range(150) == (16, 6)
    assert regions.int8_positions(10).tolist() == list(range(10))
    assert regions.int4_range(10) == (16, 0)
    assert regions.int8_positions(144).tolist() == list(range(144))
    assert regions.int4_range(144) == (16, 0)
    assert regions.int4_range(145) == (16, 1)
    assert regions.int8_positions(145).tolist() == list(range(16)) + list(range(17, 145))
    assert [regions.ring_slot(t) for t in (0, 15, 16, 143, 144, 150, 271, 272)] == \
        [0, 15, 16, 143, 16, 22, 143, 16]


def test_ring_holds_exactly_the_recent_window():
    for L in (145, 200, 1000, 4097):
        slots = [regions.ring_slot(t) for t in range(L - 128, L)]
        assert sorted(slots) == list(range(16, 144))


# ------------------------------------------------------------- composition
def exact_sources(L, D, seed):
    """K/V whose INT8 positions are INT8-exact and INT4 positions INT4-exact."""
    rng = np.random.default_rng(seed)
    x = np.zeros((L, D), np.float32)
    pos8 = set(regions.int8_positions(L).tolist())
    for t in range(L):
        if t in pos8:
            row = rng.integers(-127, 128, D).astype(np.float32)
            row[rng.integers(0, D)] = 127.0 * rng.choice([-1, 1])
        else:
            row = np.empty(D, np.float32)
            for g in range(D // 32):
                codes = rng.integers(0, 16, 32)
                codes[0], codes[1] = 0, 15
                row[g * 32:(g + 1) * 32] = codes + rng.integers(-20, 20)
        x[t] = row
    return x


@pytest.mark.parametrize("L,keep_frac", [(150, 0.5), (400, 1.0), (400, 0.3), (100, 0.0)])
def test_composition_equals_plain_attention_on_exact_data(L, keep_frac):
    D, G = 64, 4
    k, v = exact_sources(L, D, 1), exact_sources(L, D, 2)
    q = rand((G, D), 3) * 0.05
    start, n4 = regions.int4_range(L)
    keep4 = np.random.default_rng(4).random(n4) < keep_frac
    out, lse = reference.decode_group(q, k, v, keep4)
    pos = np.array(sorted(set(regions.int8_positions(L).tolist()) |
                          {start + i for i in range(n4) if keep4[i]}))
    ref_out, ref_lse = attention.attend(q, k[pos].astype(np.float64), v[pos].astype(np.float64))
    np.testing.assert_allclose(out, ref_out, rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(lse, ref_lse, rtol=1e-12)


def test_k_zero_is_sink_plus_recent_window():
    L, D = 600, 64
    k, v = rand((L, D), 8).astype(np.float32), rand((L, D), 9).astype(np.float32)
    q = rand((4, D), 10)
    out, lse = reference.decode_group(q, k, v, np.zeros(L - 144, bool))
    window = list(range(16)) + list(range(L - 128, L))
    kc, ks = quant.int8_encode(k[window])
    vc, vs = quant.int8_encode(v[window])
    ref = attention.attend(q, quant.int8_decode(kc, ks), quant.int8_decode(vc, vs))
    np.testing.assert_allclose(out, ref[0], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(lse, ref[1], rtol=1e-13)


def test_int4_region_reads_int4_and_protected_reads_int8():
    # A lossy INT4 value in a protected position must not leak into the output.
    L, D = 200, 32
    rng = np.random.default_rng(12)
    k = rng.standard_normal((L, D)).astype(np.float32)
    v = rng.standard_normal((L, D)).astype(np.float32)
    enc = reference.encode(k, v)
    kh, vh = reference.decoded(enc)
    pos8 = regions.int8_positions(L)
    k8 = quant.int8_decode(*quant.int8_encode(k[pos8]))
    k4 = quant.int4_decode(*quant.int4_encode(k))
    np.testing.assert_array_equal(kh[pos8], k8)
    mask4 = np.ones(L, bool)
    mask4[pos8] = False
    np.testing.assert_array_equal(kh[mask4], k4[mask4])
    assert not np.array_equal(k8, k4[pos8])


# ------------------------------------------------------------- pure KV4
# The KV4-RL review (section 3) compares INT8 protection against pure KV4: no
# protected positions, so every cached position is INT4 and subject to the
# keep mask. In the oracle that is n_sink = n_recent = 0.
def int4_exact_sources(L, D, seed):
    """K/V rows that the INT4 group encoding represents exactly (codes 0..15 plus an offset)."""
    rng = np.random.default_rng(seed)
    x = np.empty((L, D), np.float32)
    for t in range(L):
        for g in range(D // 32):
            codes = rng.integers(0, 16, 32)
            codes[0], codes[1] = 0, 15
            x[t, g * 32:(g + 1) * 32] = codes + rng.integers(-20, 20)
    return x


@pytest.mark.parametrize("L,keep_frac", [(1, 1.0), (40, 0.5), (300, 1.0), (300, 0.2)])
def test_pure_kv4_composition_equals_plain_attention_on_exact_data(L, keep_frac):
    D, G = 64, 2
    k, v = int4_exact_sources(L, D, 21), int4_exact_sources(L, D, 22)
    q = rand((G, D), 23) * 0.05
    keep = np.random.default_rng(24).random(L) < keep_frac
    keep[L // 2] = True  # never empty
    out, lse = reference.decode_group(q, k, v, keep, n_sink=0, n_recent=0)
    pos = np.nonzero(keep)[0]
    s = (q @ k[pos].astype(np.float64).T) / math.sqrt(D)
    mx = s.max(axis=1, keepdims=True)
    e = np.exp(s - mx)
    ref = (e @ v[pos].astype(np.float64)) / e.sum(axis=1, keepdims=True)
    np.testing.assert_allclose(out, ref, rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(lse, (mx[:, 0] + np.log(e.sum(axis=1))), rtol=1e-12)


def test_pure_kv4_reads_every_position_from_int4():
    L, D = 200, 32
    rng = np.random.default_rng(25)
    k = rng.standard_normal((L, D)).astype(np.float32)
    v = rng.standard_normal((L, D)).astype(np.float32)
    assert regions.int8_positions(L, 0, 0).shape == (0,)
    assert regions.int4_range(L, 0, 0) == (0, L)
    enc = reference.encode(k, v, 0, 0)
    kh, vh = reference.decoded(enc)
    np.testing.assert_array_equal(kh, quant.int4_decode(*quant.int4_encode(k)))
    np.testing.assert_array_equal(vh, quant.int4_decode(*quant.int4_encode(v)))
    keep = rng.random(L) < 0.3
    np.testing.assert_array_equal(reference.kept_positions(L, keep, 0, 0), np.nonzero(keep)[0])
    # the protected configuration attends the window whatever the mask says
    assert len(reference.kept_positions(L, np.zeros(L - 144, bool))) == 144


def test_pure_kv4_all_evicted_gives_empty_attention():
    L, D = 50, 32
    k = rand((L, D), 26).astype(np.float32)
    out, lse = reference.decode_group(rand((2, D), 27), k, k, np.zeros(L, bool), n_sink=0,
                                      n_recent=0)
    assert np.all(out == 0.0) and np.all(np.isneginf(lse))
