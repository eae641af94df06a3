"""Host-side checks of the C ABI (no GPU needed, no device work).

The library must load, export every function include/kvc.h declares, and
reject bad arguments with the documented status codes before touching the
device. These calls never launch a kernel.
"""
import ctypes
import os
import re

import pytest

import decode_attention_compressed_quantize_amd as kvc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(kvc.LIB_PATH):
        from decode_attention_compressed_quantize_amd import build

        build.build()
    return kvc.lib()


def declared_functions():
    src = open(os.path.join(ROOT, "include", "kvc.h")).read()
    return re.findall(r"KVC_API\s+[\w\s\*]+?\b(kvc_\w+)\s*\(", src)


def test_header_declares_the_three_entry_points():
    names = declared_functions()
    for n in ("kvc_quantize_append", "kvc_score_topk_mask", "kvc_decode_attention"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
        assert name in kvc._SIGNATURES, f"binding lacks {name}"


def test_abi_version_and_strings(lib):
    assert kvc.kvc_abi_version() == 4
    assert kvc.kvc_status_string(0) == "ok"
    assert kvc.kvc_status_string(-4) == "workspace too small"


FAKE = 0x10000  # never dereferenced: every call below fails validation first


def desc(**kw):
    d = dict(batch=2, num_kv_heads=8, head_dim=128, page_size=16, max_pages_per_seq=64,
             num_phys_pages=128, n_sink=16, n_recent=128, group=32, max_ctx=1024,
             int4_codes=FAKE, int4_meta=FAKE, int8_codes=FAKE, int8_scales=FAKE,
             block_table=FAKE, seq_lens=FAKE, keep_mask=FAKE, scores=FAKE)
    d.update(kw)
    return kvc.KvcCacheStruct(**d)


def attn(lib, c, q=FAKE, hq=32, out=FAKE, ws=FAKE, ws_bytes=1 << 40):
    return lib.kvc_decode_attention(ctypes.byref(c) if c is not None else None, q, 0, hq, 0.0,
                                    out, None, ws, ws_bytes, None)


def test_attention_argument_errors(lib):
    assert attn(lib, None) == -1
    assert attn(lib, desc(), q=None) == -1
    assert attn(lib, desc(int4_codes=None)) == -1
    assert attn(lib, desc(keep_mask=None)) == -1
    assert attn(lib, desc(head_dim=96)) == -3
    assert attn(lib, desc(page_size=32)) == -3
    assert attn(lib, desc(n_recent=64)) == -3
    assert attn(lib, desc(group=64)) == -3
    # without INT8 protection (0/0) the INT8 arrays are unused and may be NULL
    kv4 = dict(n_sink=0, n_recent=0, int8_codes=None, int8_scales=None)
    assert attn(lib, desc(**kv4), ws=None) == -4       # passes the cache checks
    assert attn(lib, desc(n_sink=16, n_recent=0)) == -3
    assert attn(lib, desc(n_sink=0, n_recent=128)) == -3
    assert attn(lib, desc(int8_codes=None)) == -1      # protected: INT8 arrays required
    c = desc(**kv4)
    assert lib.kvc_quantize_append(ctypes.byref(c), FAKE, FAKE, 0, 0, FAKE, None) == 0
    assert attn(lib, desc(max_pages_per_seq=10)) == -2
    assert attn(lib, desc(batch=0)) == -2
    assert attn(lib, desc(), hq=12) == -2          # not a multiple of Hkv
    assert attn(lib, desc(), hq=64) == -3          # G = 8 is not supported
    assert attn(lib, desc(), hq=24) == -3          # G = 3 is not supported
    assert attn(lib, desc(head_dim=64), hq=64) == -3
    assert attn(lib, desc(), q=FAKE + 2) == -3     # 16-byte alignment is required
    assert attn(lib, desc(), out=FAKE + 4) == -3
    assert attn(lib, desc(int4_codes=FAKE + 8)) == -3
    assert "aligned" in kvc.kvc_last_error()
    assert attn(lib, desc(), ws=None) == -4
    assert attn(lib, desc(), ws_bytes=16) == -4
    assert "workspace" in kvc.kvc_last_error()
    c = desc()
    assert lib.kvc_decode_attention_windowed(ctypes.byref(c), -1, FAKE, 0, 32, 0.0, FAKE, None,
                                             FAKE, 1 << 40, None) == -2
    assert lib.kvc_decode_attention_windowed(ctypes.byref(c), 100, FAKE, 0, 32, 0.0, FAKE, None,
                                             FAKE, 16, None) == -4


def test_noalloc_attention_argument_errors(lib):
    """The allocation-free entry point validates like kvc_decode_attention and refuses
    a cache whose partials exceed its fixed scratch, before any device work."""
    na = lib.kvc_decode_attention_noalloc
    assert na(None, FAKE, 0, 32, 0.0, FAKE, None, None) == -1
    assert na(ctypes.byref(desc(head_dim=96)), FAKE, 0, 32, 0.0, FAKE, None, None) == -3
    big = desc(batch=4096, max_ctx=1 << 20, max_pages_per_seq=1 << 16)
    need = lib.kvc_attention_workspace_bytes(ctypes.byref(big), 32)
    assert need > kvc.NOALLOC_SCRATCH_BYTES
    assert na(ctypes.byref(big), FAKE, 0, 32, 0.0, FAKE, None, None) == -4
    assert "scratch" in kvc.kvc_last_error()


def test_pool_argument_errors(lib):
    """Pool fields are validated before any device work."""
    c = desc(pool_capacity=100, pool=FAKE, pool_slot=FAKE, pool_header=FAKE)
    assert attn(lib, c) == -2                                   # not a multiple of 64
    c = desc(pool_capacity=128, pool=None, pool_slot=FAKE, pool_header=FAKE)
    assert attn(lib, c) == -1
    c = desc(pool_capacity=128, pool=FAKE + 4, pool_slot=FAKE, pool_header=FAKE)
    assert attn(lib, c) == -3                                   # pool must be 16-byte aligned
    ok = dict(pool=FAKE, pool_slot=FAKE, pool_header=FAKE)
    # a refresh whose budget can keep more than the pool holds: max_ctx 1024 -> 880 INT4 positions
    c = desc(pool_capacity=128, **ok)
    r = lib.kvc_score_topk_mask(ctypes.byref(c), None, None, None, 0, 0, None, 500, None, 0, None)
    assert r == -2 and "pool_capacity" in kvc.kvc_last_error()
    c = desc(pool_capacity=448, **ok)                           # 500 per mille of 880 = 440 fits
    assert lib.kvc_score_topk_mask(ctypes.byref(c), None, None, None, 0, 0, None, 500, FAKE, 16,
                                   None) == -4                  # passes the pool check
    # the block policy maintains a pool too: its whole blocks count against the capacity
    c128 = desc(pool_capacity=128, **ok)
    assert lib.kvc_score_block_mask(ctypes.byref(c128), None, None, None, 0, 0, None, 500, 16, 0,
                                    None, 0, None) == -2
    assert "pool_capacity" in kvc.kvc_last_error()
    # 500 per mille of 55 blocks of 16 = 27 blocks, 432 records: fits 448
    assert lib.kvc_score_block_mask(ctypes.byref(c), None, None, None, 0, 0, None, 500, 16, 0,
                                    FAKE, 16, None) == -4       # passes the pool check
    # a recency window of 100 positions: 7 + 1 candidate blocks, 4 kept = 64 records fit 128
    assert lib.kvc_score_block_mask(ctypes.byref(c128), None, None, None, 0, 0, None, 500, 16, 100,
                                    FAKE, 16, None) == -4
    assert lib.kvc_append_score_block_mask(ctypes.byref(c128), None, FAKE, FAKE, 0, 1, FAKE, 500,
                                           16, 0, None, 0, None) == -2
    # pool sizes and the rebuild entry point
    assert lib.kvc_pool_bytes(ctypes.byref(c)) == 2 * 8 * (448 // 32) * 40 * 128
    assert lib.kvc_pool_bytes(ctypes.byref(desc())) == 0
    assert lib.kvc_pool_build(ctypes.byref(desc()), None) == -3  # no pool
    assert lib.kvc_pool_build(None, None) == -1
    # attention over a pool needs room for the pool-mode partials too
    need = lib.kvc_attention_workspace_bytes(ctypes.byref(c), 32)
    assert need >= lib.kvc_attention_workspace_bytes(ctypes.byref(desc()), 32)
    assert attn(lib, c, ws_bytes=need - 16) == -4


def test_append_and_topk_argument_errors(lib):
    c = desc()
    r = lib.kvc_quantize_append(ctypes.byref(c), FAKE, FAKE, 0, -1, FAKE, None)
    assert r == -2
    r = lib.kvc_quantize_append(ctypes.byref(c), None, FAKE, 0, 4, FAKE, None)
    assert r == -1
    r = lib.kvc_quantize_append(ctypes.byref(c), FAKE, FAKE, 7, 4, FAKE, None)
    assert r == -3
    assert lib.kvc_quantize_append(ctypes.byref(c), FAKE, FAKE, 0, 0, FAKE, None) == 0  # no-op
    r = lib.kvc_score_topk_mask(ctypes.byref(c), None, None, None, 0, 0, None, 1001, None, 0, None)
    assert r == -2
    r = lib.kvc_score_topk_mask(ctypes.byref(desc(scores=None)), None, None, None, 0, 0, None, 500,
                                None, 0, None)
    assert r == -1
    r = lib.kvc_score_topk_mask(ctypes.byref(c), FAKE, None, FAKE, 0, 4, FAKE, 500, None, 0, None)
    assert r == -1
    r = lib.kvc_score_topk_mask(ctypes.byref(c), None, None, None, 0, 0, None, 500, FAKE, 1024, None)
    assert r == -4  # state smaller than kvc_topk_workspace_bytes
    # the fused update checks what both calls check, before any work
    fused = lib.kvc_append_score_topk_mask
    assert fused(None, FAKE, FAKE, FAKE, 0, 1, FAKE, 500, None, 0, None) == -1
    assert fused(ctypes.byref(c), FAKE, FAKE, FAKE, 0, 1, FAKE, 1001, None, 0, None) == -2
    assert fused(ctypes.byref(c), FAKE, FAKE, FAKE, 0, -1, FAKE, 500, None, 0, None) == -2
    assert fused(ctypes.byref(c), FAKE, None, FAKE, 0, 1, FAKE, 500, None, 0, None) == -1
    assert fused(ctypes.byref(c), FAKE, FAKE, FAKE, 7, 1, FAKE, 500, None, 0, None) == -3
    assert fused(ctypes.byref(c), FAKE, FAKE, FAKE, 0, 1, FAKE, 500, FAKE, 1024, None) == -4
    assert fused(ctypes.byref(desc(scores=None)), FAKE, FAKE, FAKE, 0, 1, FAKE, 500, None, 0,
                 None) == -1
    assert fused(ctypes.byref(desc(int8_codes=None)), FAKE, FAKE, FAKE, 0, 1, FAKE, 500, None, 0,
                 None) == -1
    fb = lib.kvc_append_score_block_mask
    assert fb(None, FAKE, FAKE, FAKE, 0, 1, FAKE, 500, 16, 0, None, 0, None) == -1
    assert fb(ctypes.byref(c), FAKE, FAKE, FAKE, 0, 1, FAKE, 500, 24, 0, None, 0, None) == -3
    assert fb(ctypes.byref(c), FAKE, FAKE, FAKE, 0, 1, FAKE, 500, 16, -1, None, 0, None) == -2
    assert fb(ctypes.byref(c), FAKE, FAKE, FAKE, 0, 1, FAKE, -1, 16, 0, None, 0, None) == -2
    assert fb(ctypes.byref(c), FAKE, FAKE, FAKE, 0, 1, FAKE, 500, 16, 0, FAKE, 64, None) == -4


def test_workspace_size_covers_every_split(lib):
    # (m, l, o[D]) per query head for every INT4 chunk of at most 8192
    # positions plus the INT8 partial, and at most 256 partials
    for max_ctx in (1, 144, 145, 4096, 131072, 2089088):
        c = desc(max_ctx=max_ctx, max_pages_per_seq=(max_ctx + 15) // 16)
        n = lib.kvc_attention_workspace_bytes(ctypes.byref(c), 32)
        counters = 0
        per_split = 2 * 32 * (128 + 2) * 4
        assert (n - counters) % per_split == 0
        nparts = (n - counters) // per_split
        assert nparts >= 2
        end4 = max(0, max_ctx - 128) if max_ctx > 144 else 0
        assert (nparts - 1) * 8192 >= end4
        assert nparts <= 256
    assert lib.kvc_attention_workspace_bytes(ctypes.byref(desc(head_dim=96)), 32) == 0
    assert lib.kvc_topk_workspace_bytes(ctypes.byref(desc())) == 2 * 8 * 1056
    assert lib.kvc_topk_workspace_bytes(ctypes.byref(desc(head_dim=96))) == 0


def test_block_mask_argument_errors(lib):
    def call(c, budget=500, block=16, window=0, mlp=None, n_max=0, ws=None, ws_bytes=0):
        return lib.kvc_score_block_mask(ctypes.byref(c), mlp, None, None, 0, n_max, None, budget,
                                        block, window, ws, ws_bytes, None)

    assert call(desc(), block=8) == -3
    assert call(desc(), block=48) == -3
    assert "16, 32 or 64" in kvc.kvc_last_error()
    assert call(desc(), budget=1001) == -2
    assert call(desc(), budget=-1) == -2
    assert call(desc(), window=-1) == -2
    assert call(desc(scores=None)) == -1
    assert call(desc(keep_mask=None)) == -1
    assert call(desc(), mlp=FAKE, n_max=4) == -1   # MLP without K/V rows
    need = lib.kvc_block_workspace_bytes(ctypes.byref(desc()), 16)
    assert call(desc(), ws=FAKE, ws_bytes=need - 16) == -4
    assert "state" in kvc.kvc_last_error()
    assert call(desc(), ws=FAKE + 4, ws_bytes=need) == -3
    # more than 131072 blocks per sequence
    big = 131072 * 16 + 1
    assert call(desc(max_ctx=big, max_pages_per_seq=(big + 15) // 16)) == -3


def test_tier_argument_errors(lib):
    c = desc(num_host_pages=4)            # host pool pointers missing
    assert lib.kvc_copy_pages(ctypes.byref(c), FAKE, FAKE, 1, None) == -1
    assert attn(lib, c) == -1
    assert attn(lib, desc(num_host_pages=-1)) == -2
    ok = desc(num_host_pages=4, int4_codes_host=FAKE, int4_meta_host=FAKE)
    assert attn(lib, ok, ws=None) == -4   # passes the cache checks
    assert lib.kvc_copy_pages(ctypes.byref(ok), FAKE, FAKE, 0, None) == 0
    assert lib.kvc_copy_pages(ctypes.byref(ok), None, FAKE, 3, None) == -1
    assert lib.kvc_find_pages(ctypes.byref(ok), 2, FAKE, 8, FAKE, None) == -2
    assert lib.kvc_find_pages(ctypes.byref(ok), 0, None, 8, FAKE, None) == -1
    assert attn(lib, desc(num_host_pages=4, int4_codes_host=FAKE + 4, int4_meta_host=FAKE)) == -3


def test_block_workspace_size(lib):
    # 64-byte header + one 4-byte key per 16 INT4-region positions, rounded up
    # to 16 bytes; the same for every block size
    for max_ctx in (1, 144, 145, 1024, 131072 + 26):
        c = desc(max_ctx=max_ctx, max_pages_per_seq=(max_ctx + 15) // 16)
        n4 = max(0, max_ctx - 144)
        keys = (n4 + 15) // 16
        stride = 64 + (keys + 3) // 4 * 16
        for B in (16, 32, 64):
            assert lib.kvc_block_workspace_bytes(ctypes.byref(c), B) == 2 * 8 * stride
    assert lib.kvc_block_workspace_bytes(ctypes.byref(desc()), 8) == 0
    assert lib.kvc_block_workspace_bytes(ctypes.byref(desc(head_dim=96)), 16) == 0


def ddesc(**kw):
    d = dict(batch=2, num_kv_heads=8, head_dim=128, page_size=16, max_pages_per_seq=64,
             num_phys_pages=128, max_ctx=1024, reserved=0, kv=FAKE, block_table=FAKE, seq_lens=FAKE)
    d.update(kw)
    return kvc.KvcDenseCacheStruct(**d)


def dattn(lib, c, q=FAKE, hq=32, out=FAKE, ws=FAKE, ws_bytes=1 << 40):
    return lib.kvc_dense_decode_attention(ctypes.byref(c) if c is not None else None, q, 0, hq, 0.0,
                                          out, None, ws, ws_bytes, None)


def test_dense_argument_errors(lib):
    assert dattn(lib, None) == -1
    assert dattn(lib, ddesc(kv=None)) == -1
    assert dattn(lib, ddesc(block_table=None)) == -1
    assert dattn(lib, ddesc(), q=None) == -1
    assert dattn(lib, ddesc(head_dim=96)) == -3
    assert dattn(lib, ddesc(page_size=32)) == -3
    assert dattn(lib, ddesc(max_pages_per_seq=10)) == -2
    assert dattn(lib, ddesc(batch=0)) == -2
    assert dattn(lib, ddesc(), hq=12) == -2
    assert dattn(lib, ddesc(), hq=64) == -3
    assert dattn(lib, ddesc(kv=FAKE + 2)) == -3
    assert dattn(lib, ddesc(), q=FAKE + 4) == -3
    assert dattn(lib, ddesc(), ws=None) == -4
    assert dattn(lib, ddesc(), ws_bytes=16) == -4
    big = 256 * 8192 + 1
    assert dattn(lib, ddesc(max_ctx=big, max_pages_per_seq=(big + 15) // 16)) == -3
    c = ddesc()
    app = lib.kvc_dense_append
    assert app(None, FAKE, FAKE, 0, 1, FAKE, None) == -1
    assert app(ctypes.byref(c), FAKE, FAKE, 0, -1, FAKE, None) == -2
    assert app(ctypes.byref(c), None, FAKE, 0, 1, FAKE, None) == -1
    assert app(ctypes.byref(c), FAKE, FAKE, 7, 1, FAKE, None) == -3
    assert app(ctypes.byref(c), FAKE + 2, FAKE, 0, 1, FAKE, None) == -3
    assert app(ctypes.byref(c), FAKE, FAKE, 0, 0, FAKE, None) == 0  # no-op


def test_dense_workspace_size(lib):
    # one (m, l, o[D]) partial per query head per chunk; chunks of at most 8192 positions,
    # at most 256 of them, and about 512 chunk workgroups once the work allows it
    for max_ctx, batch in ((1, 1), (100, 2), (4096, 64), (131072, 4), (131072 + 32, 4),
                           (256 * 8192, 1)):
        c = ddesc(max_ctx=max_ctx, batch=batch, max_pages_per_seq=(max_ctx + 15) // 16)
        n = lib.kvc_dense_attention_workspace_bytes(ctypes.byref(c), 32)
        per_split = batch * 32 * (128 + 2) * 4
        assert n % per_split == 0
        nsplit = n // per_split
        assert 1 <= nsplit <= 256
        assert nsplit * 8192 >= max_ctx
    c = ddesc(max_ctx=131072, batch=4, max_pages_per_seq=8192)
    assert lib.kvc_dense_attention_workspace_bytes(ctypes.byref(c), 32) == 4 * 32 * 130 * 4 * 16
    assert lib.kvc_dense_attention_workspace_bytes(ctypes.byref(ddesc(head_dim=96)), 32) == 0
    assert lib.kvc_dense_attention_workspace_bytes(ctypes.byref(ddesc()), 12) == 0


def test_read_probe_argument_errors(lib):
    probe = lib.kvc_stream_read_probe
    assert probe(None, 0, None, None) == 0            # nothing to read
    assert probe(None, 64, FAKE, None) == -1
    assert probe(FAKE, 64, None, None) == -1
    assert probe(FAKE + 4, 64, FAKE, None) == -3      # 16-byte alignment
    assert probe(FAKE, 60, FAKE, None) == -3          # whole 16-byte pieces
    assert probe(FAKE, 64, FAKE + 2, None) == -3      # out is written atomically
