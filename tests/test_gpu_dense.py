"""GPU parity of the dense bfloat16 baseline (kvc_dense_append, kvc_dense_decode_attention)
against the CPU oracle (oracle.dense).

Stored rows are compared bit for bit with the oracle's bfloat16 rounding; attention output
and LSE within max-abs 1e-4, rel-L2 2e-5 and LSE max-abs 1e-4. The kernel's logits use
the query as two bfloat16 parts (~16 significant bits) against exact bfloat16 keys with
float32 accumulation, and P.V is float32: the error budget is about 2^-18 of sum |q_d k_d|
times the scale in a logit (~3e-5 at D = 128 for unit normal rows) plus float32 rounding,
so the bounds hold with margin (observed errors are printed).
"""
import numpy as np
import pytest
import torch

import workloads as W
from decode_attention_compressed_quantize_amd import (DenseCache, dense_workspace,
                                                      kvc_dense_append, kvc_dense_decode_attention)
from decode_attention_compressed_quantize_amd.workload_cache import DenseLayerCache
from kvc_testlib import source_np, to_f32
from oracle import dense

pytestmark = pytest.mark.gpu

ATOL, RTOL2, LTOL = 1e-4, 2e-5, 1e-4


def check(out, lse, ref_out, ref_lse, what):
    out = np.asarray(out, np.float64)
    err = np.abs(out - ref_out).max()
    rel = np.linalg.norm(out - ref_out) / max(np.linalg.norm(ref_out), 1e-30)
    empty = np.isneginf(ref_lse)
    assert np.array_equal(np.isneginf(lse), empty), f"{what}: lse -inf mismatch"
    lerr = np.abs(lse[~empty] - ref_lse[~empty]).max() if (~empty).any() else 0.0
    print(f"  {what}: max-abs {err:.2e} rel-L2 {rel:.2e} lse {lerr:.2e}", flush=True)
    assert err <= ATOL and rel <= RTOL2 and lerr <= LTOL, what


def oracle_pair(w, layer, b, kvh, L, q, scale=None, skip=None):
    """Oracle (out [G][D], lse [G]) of kv head kvh of sequence b over positions [0, L)
    minus the positions in ``skip``."""
    k = source_np(w, layer, "K", b, L, kvh)
    v = source_np(w, layer, "V", b, L, kvh)
    if skip is not None and len(skip):
        keep = np.ones(L, bool)
        keep[skip] = False
        k, v = k[keep], v[keep]
    G = w.group_size
    qh = to_f32(q[b, kvh * G:(kvh + 1) * G]).astype(np.float64)
    return dense.decode_group(qh, k, v, w.src_dtype, scale)


def q_np(q):
    if q.dtype == torch.bfloat16:
        return q.view(torch.int16).cpu().numpy().view(np.uint16)
    return q.cpu().numpy()


def run(lc, q, scale=0.0):
    w = lc.w
    out = torch.full((w.batch, w.q_heads, w.head_dim), 7.0, dtype=torch.float32, device="cuda")
    lse = torch.full((w.batch, w.q_heads), 7.0, dtype=torch.float32, device="cuda")
    kvc_dense_decode_attention(lc.cache, q, out, lse, lc.workspace(), softmax_scale=scale)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy()


CASES = [
    # name, batch, Hq, Hkv, D, lengths, src
    ("d128g4", 3, 8, 2, 128, (1, 700, 2049), "bf16"),
    ("d128g2f32", 2, 4, 2, 128, (1500, 33), "f32"),
    ("d64g1", 2, 2, 2, 64, (257, 3000), "bf16"),
    ("d64g4f32", 2, 8, 2, 64, (96, 4100), "f32"),
    ("zero_len", 3, 8, 2, 128, (0, 40, 0), "bf16"),
]


@pytest.mark.parametrize("name,B,Hq,Hkv,D,lens,src", CASES, ids=[c[0] for c in CASES])
def test_dense_attention_every_pair(name, B, Hq, Hkv, D, lens, src):
    w = W.Workload(f"dense_{name}", B, Hq, Hkv, D, ctx_list=lens, src_dtype=src)
    print(f"dense parity {name}", flush=True)
    lc = DenseLayerCache(w)
    q = lc.queries(0)
    out, lse = run(lc, q)
    qn = q_np(q)
    G = w.group_size
    for b in range(B):
        for h in range(Hkv):
            ref_out, ref_lse = oracle_pair(w, 0, b, h, int(lens[b]), qn)
            check(out[b, h * G:(h + 1) * G], lse[b, h * G:(h + 1) * G], ref_out, ref_lse,
                  f"{name} b={b} h={h} L={lens[b]}")


def test_dense_stored_rows_are_bf16_of_the_sources():
    for src in ("f32", "bf16"):
        w = W.Workload(f"dense_rows_{src}", 2, 4, 2, 64, ctx_list=(50, 17), src_dtype=src)
        lc = DenseLayerCache(w)
        kv = lc.cache.kv.cpu().numpy().view(np.uint16)
        table = lc.table_np
        for b in range(w.batch):
            L = int(w.lengths()[b])
            npg = (L + 15) // 16
            for h in range(w.kv_heads):
                rows = kv[table[b, :npg], h].reshape(npg * 16, 2, w.head_dim)[:L]
                for which, idx in (("K", 0), ("V", 1)):
                    want = dense.store_rows(source_np(w, 0, which, b, L, h), src)
                    got = W.bf16_bits_to_f32(rows[:, idx])
                    np.testing.assert_array_equal(got.view(np.uint32), want.view(np.uint32),
                                                  err_msg=f"{src} {which} b={b} h={h}")


def test_dense_out_of_range_pages_are_skipped():
    w = W.Workload("dense_badpages", 2, 8, 2, 128, ctx_list=(1000, 600), src_dtype="bf16")
    lc = DenseLayerCache(w)
    table = lc.table_np.copy()
    table[0, 3] = -1
    table[0, 40] = lc.num_pages + 5
    table[1, 0] = 1 << 30
    lc.table.copy_(torch.from_numpy(table))
    q = lc.queries(1)
    out, lse = run(lc, q)
    qn = q_np(q)
    skips = {0: list(range(48, 64)) + list(range(640, 656)), 1: list(range(0, 16))}
    for b in range(2):
        for h in range(2):
            ref_out, ref_lse = oracle_pair(w, 0, b, h, int(w.lengths()[b]), qn,
                                           skip=np.array(skips[b]))
            check(out[b, h * 4:(h + 1) * 4], lse[b, h * 4:(h + 1) * 4], ref_out, ref_lse,
                  f"badpages b={b} h={h}")


def test_dense_decode_steps_append_then_attend():
    w = W.Workload("dense_steps", 2, 8, 2, 128, ctx_list=(300, 1023), src_dtype="bf16",
                   decode_steps=4)
    lc = DenseLayerCache(w)
    lens = w.lengths().copy()
    one = torch.ones(w.batch, dtype=torch.int32, device="cuda")
    for s in range(3):
        k_new = W.kv_rows_torch(w, 0, "K", lens, "cuda")[:, None]
        v_new = W.kv_rows_torch(w, 0, "V", lens, "cuda")[:, None]
        lens += 1
        lc.seq_lens.add_(1)
        lc.append(k_new, v_new, one)
        q = lc.queries(s + 1)
        out, lse = run(lc, q)
        qn = q_np(q)
        for b in range(w.batch):
            for h in range(w.kv_heads):
                ref_out, ref_lse = oracle_pair(w, 0, b, h, int(lens[b]), qn)
                check(out[b, h * 4:(h + 1) * 4], lse[b, h * 4:(h + 1) * 4], ref_out, ref_lse,
                      f"step {s} b={b} h={h} L={lens[b]}")


def test_dense_explicit_scale():
    w = W.Workload("dense_scale", 1, 4, 1, 128, ctx_list=(777,), src_dtype="f32")
    lc = DenseLayerCache(w)
    q = lc.queries(0)
    out, lse = run(lc, q, scale=0.05)
    ref_out, ref_lse = oracle_pair(w, 0, 0, 0, 777, q_np(q), scale=0.05)
    check(out[0], lse[0], ref_out, ref_lse, "scale 0.05")


def test_dense_full_size_sampled_pairs():
    """The 128K benchmark shape (4 x 131072, 32 query / 8 kv heads) in the benchmark's
    launch configuration; the oracle checks a sample of (sequence, kv head) pairs."""
    w = W.Workload("dense_long128k", 4, 32, 8, 128, ctx=131072, src_dtype="bf16", decode_steps=32)
    print("dense full size: building", flush=True)
    lc = DenseLayerCache(w)
    q = lc.queries(0)
    out, lse = run(lc, q)
    qn = q_np(q)
    for b, h in ((0, 0), (1, 5), (2, 3), (3, 7)):
        ref_out, ref_lse = oracle_pair(w, 0, b, h, 131072, qn)
        check(out[b, h * 4:(h + 1) * 4], lse[b, h * 4:(h + 1) * 4], ref_out, ref_lse,
              f"long128k b={b} h={h}")
    assert np.isfinite(out).all() and np.isfinite(lse).all()
