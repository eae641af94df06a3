"""Attention at the longest context each cache accepts, where the merge combines
the most partials (255 INT4 chunks plus the INT8 region; 256 dense chunks).
Compared with the CPU oracle like the other parity tests."""
import numpy as np
import pytest
import torch

import workloads as W
import decode_attention_compressed_quantize_amd as kvc
from decode_attention_compressed_quantize_amd.workload_cache import DenseLayerCache, LayerCache
from kvc_testlib import assert_attention_close, keep4_from_mask, oracle_heads, source_np, to_f32
from oracle import dense

pytestmark = pytest.mark.gpu


def q_np(q):
    return q.view(torch.int16).cpu().numpy().view(np.uint16) if q.dtype == torch.bfloat16 else q.cpu().numpy()


def test_compressed_attention_at_max_context():
    L = 255 * 8192 + 128  # 2,089,088
    w = W.Workload("max_ctx_int4", 1, 4, 1, 64, ctx=L, src_dtype="bf16", mask="bernoulli")
    print(f"max-context INT4 cache: building L={L}", flush=True)
    lc = LayerCache(w, keep_sources=False)
    ws = lc.workspace()
    assert ws.numel() * 4 == kvc.kvc_attention_workspace_bytes(lc.cache, 4)
    q = lc.queries(0)
    out = torch.empty((1, 4, 64), dtype=torch.float32, device="cuda")
    lse = torch.empty((1, 4), dtype=torch.float32, device="cuda")
    kvc.kvc_decode_attention(lc.cache, q, out, lse, ws)
    torch.cuda.synchronize()
    mask = lc.cache.keep_mask.cpu().numpy()
    keep4 = keep4_from_mask(mask[0, 0], L)
    ref_out, ref_lse = oracle_heads(w, 0, 0, 0, L, keep4, q_np(q)[0])
    err = assert_attention_close(out[0].cpu().numpy(), lse[0].cpu().numpy(), ref_out, ref_lse,
                                 "max context")
    print(f"  max-abs {err[0]:.2e} rel-L2 {err[1]:.2e} lse {err[2]:.2e}", flush=True)


def test_dense_attention_at_max_context():
    L = 256 * 8192  # 2,097,152
    w = W.Workload("max_ctx_dense", 1, 4, 1, 64, ctx=L, src_dtype="bf16")
    print(f"max-context dense cache: building L={L}", flush=True)
    lc = DenseLayerCache(w)
    q = lc.queries(0)
    out = torch.empty((1, 4, 64), dtype=torch.float32, device="cuda")
    lse = torch.empty((1, 4), dtype=torch.float32, device="cuda")
    kvc.kvc_dense_decode_attention(lc.cache, q, out, lse, lc.workspace())
    torch.cuda.synchronize()
    k = source_np(w, 0, "K", 0, L, 0)
    v = source_np(w, 0, "V", 0, L, 0)
    ref_out, ref_lse = dense.decode_group(to_f32(q_np(q)[0]).astype(np.float64), k, v, "bf16")
    o = out[0].cpu().numpy().astype(np.float64)
    err = np.abs(o - ref_out).max()
    rel = np.linalg.norm(o - ref_out) / np.linalg.norm(ref_out)
    lerr = np.abs(lse[0].cpu().numpy() - ref_lse).max()
    print(f"  dense max-abs {err:.2e} rel-L2 {rel:.2e} lse {lerr:.2e}", flush=True)
    assert err <= 1e-4 and rel <= 2e-5 and lerr <= 1e-4
