"""GPU test of kvc_decode_attention_noalloc: the allocation-free variant of
kvc_decode_attention (its partials live in the library's per-GPU scratch).

Calls in a row through the C ABI, the second on a smaller cache (so it
reads a scratch that still holds the first call's partials), the third on a
cache with a kept-record pool, each compared
with kvc_decode_attention on the same inputs: the same kernels and the same
split plan run, so outputs and LSE must be bit-identical; and both are
checked against the CPU oracle on sampled (sequence, kv head) pairs.
"""
import numpy as np
import pytest

import workloads as W

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _cases():
    """(workload, kept-record pool): mask mode twice (the second smaller), then
    pool mode, whose last workgroup per (sequence, kv head) merges the
    partials from the scratch in the same launch."""
    big = W.Workload("noalloc_big", 8, 32, 8, 128, ctx=6000, mask="mlp", budget_permille=500)
    small = W.Workload("noalloc_small", 3, 8, 4, 64, ctx_list=(700, 145, 1999), mask="mlp",
                       budget_permille=300, src_dtype="f32")
    pooled = W.Workload("noalloc_pool", 4, 32, 8, 128, ctx_list=(9000, 145, 3000, 20000), mask="mlp",
                        budget_permille=300)
    return [(big, False), (small, False), (pooled, True)]


def test_noalloc_matches_workspace_entry_point_twice():
    import decode_attention_compressed_quantize_amd as kvc
    from decode_attention_compressed_quantize_amd.workload_cache import LayerCache
    from kvc_testlib import assert_attention_close, keep4_from_mask, oracle_heads

    kvc.lib()
    for i, (w, pool) in enumerate(_cases()):
        print(f"noalloc call {i}: {w.name} B={w.batch} Hq={w.q_heads} Hkv={w.kv_heads} "
              f"D={w.head_dim} pool={pool}", flush=True)
        lc = LayerCache(w, pool=pool)
        q = lc.queries(0)
        need = kvc.kvc_attention_workspace_bytes(lc.cache, w.q_heads)
        assert 0 < need <= kvc.NOALLOC_SCRATCH_BYTES
        out_ws = torch.full((w.batch, w.q_heads, w.head_dim), float("nan"), device="cuda")
        lse_ws = torch.full((w.batch, w.q_heads), float("nan"), device="cuda")
        out_na = torch.full_like(out_ws, float("nan"))
        lse_na = torch.full_like(lse_ws, float("nan"))
        kvc.kvc_decode_attention(lc.cache, q, out_ws, lse_ws, lc.workspace())
        kvc.kvc_decode_attention_noalloc(lc.cache, q, out_na, lse_na)
        torch.cuda.synchronize()
        assert torch.equal(out_na, out_ws), f"{w.name}: outputs differ"
        assert torch.equal(lse_na, lse_ws), f"{w.name}: lse differ"
        # and against the oracle on a few pairs
        mask = lc.cache.keep_mask.cpu().numpy()
        qn = q.float().cpu().numpy()
        G = w.group_size
        for b in range(w.batch):
            kvh = (3 * b) % w.kv_heads
            L = int(lc.lengths[b])
            keep4 = keep4_from_mask(mask[b, kvh], L)
            ref_out, ref_lse = oracle_heads(w, 0, b, kvh, L, keep4, qn[b, kvh * G:(kvh + 1) * G])
            assert_attention_close(out_na[b, kvh * G:(kvh + 1) * G].cpu().numpy(),
                                   lse_na[b, kvh * G:(kvh + 1) * G].cpu().numpy(), ref_out, ref_lse,
                                   f"{w.name} b={b} kvh={kvh}")
        del lc
