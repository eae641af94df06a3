"""Test-side helpers: read GPU cache buffers through the documented layout and
compute the oracle's expectation for one (sequence, kv head).

The layout readers follow the memory-layout section of include/kvc.h; they
share no code with the library.
"""
from __future__ import annotations

import math

import numpy as np

import workloads as W
from oracle import policy, quant, reference, regions

D_GROUP = 32


def prot(w):
    """(n_sink, n_recent) of a workload: the INT8-protected counts, or 0, 0 for pure KV4."""
    return (regions.N_SINK, regions.N_RECENT) if w.protect else (0, 0)


def to_f32(src):
    """Source values (bf16 bits uint16 or float32) as float32."""
    if src.dtype == np.uint16:
        return W.bf16_bits_to_f32(src)
    return np.asarray(src, np.float32)


def source_np(w, layer, which, b, L, kvh):
    return to_f32(W.kv_source_np(w, layer, which, b, 0, L, kvh=kvh))


def unpage_int4(codes, meta, table, b, kvh, L):
    """GPU INT4 buffers -> (K codes [L][D/2], V codes [L][D/2], meta [L][2][D/32][2] uint16).

    meta[..., 0, g, 0] is the K scale of group g, [..., 0, g, 1] the K min,
    [..., 1, g, 0] the V scale and [..., 1, g, 1] the V min.
    """
    npg = (L + 15) // 16
    pages = table[b, :npg]
    c = codes[pages, kvh].reshape(npg * 16, 2, codes.shape[-1])[:L]
    m = meta[pages, kvh].reshape(npg * 16, 2, meta.shape[-2], 2)[:L]
    return c[:, 0], c[:, 1], m.view(np.uint16)


def int8_slot_rows(codes8, scales8, b, kvh, L):
    """GPU INT8 buffers in position order of the protected positions."""
    pos = regions.int8_positions(L)
    slots = np.array([regions.ring_slot(int(t)) for t in pos], dtype=np.int64)
    c = codes8[b, kvh, slots]           # [n8][2][D]
    s = scales8[b, kvh, slots]          # [n8][2]
    return pos, c[:, 0], c[:, 1], s[:, 0], s[:, 1]


def mask_bits(words_row, L):
    w = np.asarray(words_row).view(np.uint32).astype(np.uint64)
    bits = ((w[:, None] >> np.arange(32, dtype=np.uint64)) & np.uint64(1)).reshape(-1)
    return bits[:L].astype(bool)


def keep4_from_mask(words_row, L, n_sink=regions.N_SINK, n_recent=regions.N_RECENT):
    start, n4 = regions.int4_range(L, n_sink, n_recent)
    return mask_bits(words_row, L)[start:start + n4]


def check_codes(w, layer, b, kvh, L, cpu):
    """Bit-exact comparison of one (sequence, kv head) of GPU buffers with the oracle."""
    k = source_np(w, layer, "K", b, L, kvh)
    v = source_np(w, layer, "V", b, L, kvh)
    enc = reference.encode(k, v, *prot(w))
    kc, vc, meta = unpage_int4(cpu["int4_codes"], cpu["int4_meta"], cpu["table"], b, kvh, L)
    np.testing.assert_array_equal(kc, quant.pack_nibbles(enc["k4"]), err_msg=f"K INT4 codes b={b} h={kvh}")
    np.testing.assert_array_equal(vc, quant.pack_nibbles(enc["v4"]), err_msg=f"V INT4 codes b={b} h={kvh}")
    np.testing.assert_array_equal(meta[:, 0, :, 0], enc["k4_scale"].view(np.uint16), err_msg="K scale")
    np.testing.assert_array_equal(meta[:, 0, :, 1], enc["k4_min"].view(np.uint16), err_msg="K min")
    np.testing.assert_array_equal(meta[:, 1, :, 0], enc["v4_scale"].view(np.uint16), err_msg="V scale")
    np.testing.assert_array_equal(meta[:, 1, :, 1], enc["v4_min"].view(np.uint16), err_msg="V min")
    if not w.protect:  # no INT8 side cache
        return enc
    pos, k8, v8, ks8, vs8 = int8_slot_rows(cpu["int8_codes"], cpu["int8_scales"], b, kvh, L)
    np.testing.assert_array_equal(k8, enc["k8"], err_msg="K INT8 codes")
    np.testing.assert_array_equal(v8, enc["v8"], err_msg="V INT8 codes")
    np.testing.assert_array_equal(ks8.view(np.uint32), enc["k8_scale"].view(np.uint32), err_msg="K INT8 scale")
    np.testing.assert_array_equal(vs8.view(np.uint32), enc["v8_scale"].view(np.uint32), err_msg="V INT8 scale")
    return enc


def oracle_heads(w, layer, b, kvh, L, keep4, q_heads, scale=None):
    """Oracle (out [G][D], lse [G]) for the query heads of kv head ``kvh``."""
    k = source_np(w, layer, "K", b, L, kvh)
    v = source_np(w, layer, "V", b, L, kvh)
    q = to_f32(q_heads).astype(np.float64)
    return reference.decode_group(q, k, v, keep4, scale, *prot(w))


def assert_attention_close(out, lse, ref_out, ref_lse, what=""):
    """max-abs 2e-3 and rel-L2 1e-3 on the output, max-abs 2e-3 on the LSE."""
    out = np.asarray(out, np.float64)
    ref_out = np.asarray(ref_out, np.float64)
    err = np.abs(out - ref_out).max()
    rel = np.linalg.norm(out - ref_out) / max(np.linalg.norm(ref_out), 1e-30)
    lse = np.asarray(lse, np.float64)
    ref_lse = np.asarray(ref_lse, np.float64)
    # nothing attended (possible without INT8 protection): lse = -inf on both sides
    empty = np.isneginf(ref_lse)
    assert np.array_equal(np.isneginf(lse), empty), f"{what} lse -inf where the oracle has none"
    lerr = np.abs(lse[~empty] - ref_lse[~empty]).max() if (~empty).any() else 0.0
    assert err <= 2e-3, f"{what} max-abs {err:.3e}"
    assert rel <= 1e-3, f"{what} rel-L2 {rel:.3e}"
    assert lerr <= 2e-3, f"{what} lse max-abs {lerr:.3e}"
    return err, rel, lerr


POOL_MAGIC = 0x4B565031


def unpack_pool(pool_pair, D, n):
    """Records of slots [0, n) of one (sequence, kv head)'s pool (uint8 [tiles][40*D]) ->
    (K codes [n][D/2], V codes [n][D/2], meta uint16 [n][2][D/32][2]).

    Tile layout (32 records): K codes as pieces (t // 16, s, t % 16) of D/8 bytes
    (bytes [s*D/8, (s+1)*D/8) of token t), then K meta, V codes and V meta as
    dwords indexed [r(t)][g or d][t % 4] with r(t) = 4 (t // 16) + (t % 16) // 4."""
    NG, SB, VD = D // 32, D // 8, D // 8
    nt = (n + 31) // 32
    tiles = np.ascontiguousarray(pool_pair[:nt]).reshape(nt, 40 * D)
    t = np.arange(32)
    r_t = ((t >> 4) << 2) + ((t & 15) >> 2)
    j_t = t & 3
    kc = tiles[:, :16 * D].reshape(nt, 2, 4, 16, SB).transpose(0, 1, 3, 2, 4).reshape(nt, 32, 4 * SB)
    km = tiles[:, 16 * D:20 * D].copy().view(np.uint32).reshape(nt, 8, NG, 4)
    vc = tiles[:, 20 * D:36 * D].copy().view(np.uint32).reshape(nt, 8, VD, 4)
    vm = tiles[:, 36 * D:40 * D].copy().view(np.uint32).reshape(nt, 8, NG, 4)
    kmeta = km[:, r_t, :, j_t].transpose(1, 0, 2)   # [nt][32][NG]
    vcode = vc[:, r_t, :, j_t].transpose(1, 0, 2)   # [nt][32][VD]
    vmeta = vm[:, r_t, :, j_t].transpose(1, 0, 2)
    kcodes = kc.reshape(nt * 32, D // 2)[:n]
    vcodes = np.ascontiguousarray(vcode.reshape(nt * 32, VD)).view(np.uint8).reshape(nt * 32, D // 2)[:n]
    meta = np.stack([kmeta.reshape(nt * 32, NG), vmeta.reshape(nt * 32, NG)], axis=1)[:n]
    return kcodes, vcodes, np.ascontiguousarray(meta).view(np.uint16).reshape(n, 2, NG, 2)


def check_pool(cpu, b, kvh, L, keep4, D, n_sink=regions.N_SINK):
    """The pool of one (sequence, kv head) holds exactly the kept INT4 records, bit for bit:
    header (count, length, magic), a slot per kept position covering [0, count) once, and
    each slot's record equal to the paged record of its position. Returns the count."""
    hdr = cpu["pool_header"][b, kvh]
    kept = n_sink + np.flatnonzero(np.asarray(keep4, bool))
    n = kept.size
    assert int(hdr[2]) & 0xFFFFFFFF == POOL_MAGIC, f"pool b={b} h={kvh}: not valid"
    assert int(hdr[1]) == L, f"pool b={b} h={kvh}: length {int(hdr[1])}, expected {L}"
    assert int(hdr[0]) == n, f"pool b={b} h={kvh}: {int(hdr[0])} records, mask keeps {n}"
    assert int(hdr[3]) == 0, f"pool b={b} h={kvh}: workgroup counter left at {int(hdr[3])}"
    if n == 0:
        return 0
    maps = cpu["pool_slot"][b, kvh]
    max_ctx = maps.shape[0] - cpu["pool"].shape[2] * 32
    slots = maps[kept].astype(np.int64)
    assert np.array_equal(np.sort(slots), np.arange(n)), f"pool b={b} h={kvh}: slots are not 0..{n - 1}"
    np.testing.assert_array_equal(maps[max_ctx + slots], kept, err_msg=f"pool b={b} h={kvh}: slot->position map")
    kc, vc, meta = unpage_int4(cpu["int4_codes"], cpu["int4_meta"], cpu["table"], b, kvh, L)
    pk, pv, pm = unpack_pool(cpu["pool"][b, kvh], D, n)
    np.testing.assert_array_equal(pk[slots], kc[kept], err_msg=f"pool K codes b={b} h={kvh}")
    np.testing.assert_array_equal(pv[slots], vc[kept], err_msg=f"pool V codes b={b} h={kvh}")
    np.testing.assert_array_equal(pm[slots], meta[kept], err_msg=f"pool meta b={b} h={kvh}")
    return n
