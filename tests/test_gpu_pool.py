"""GPU parity of the kept-record pool and of attention in pool mode.

The pool must hold exactly the INT4 records the keep mask keeps, bit for bit
(checked through an independent reader of its tile layout against the paged
store), after a rebuild from a caller-written mask, after a full refresh and
after every incremental decode step; attention over it must meet the same
tolerances against the float64 oracle as attention through the mask. Also:
the error word, and the rollback contract (re-append the recent window after
shrinking a length).
"""
import numpy as np
import pytest

import workloads as W
from kvc_testlib import (assert_attention_close, check_pool, keep4_from_mask, mask_bits,
                         oracle_heads, prot)
from oracle import policy, regions
from test_gpu_parity import LayerCache, check_workload, cpu_buffers, kvc, run_attention, sample_pairs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _needs_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


SMALL = {
    "tiny": W.WORKLOADS["tiny"],
    "uniform_small": W.WORKLOADS["uniform4k"].replace(name="uniform_small", batch=3, ctx=1000),
    "edges": W.WORKLOADS["longtail"].replace(name="edges", batch=10, ctx_range=None,
                                             ctx_list=(1, 16, 17, 100, 144, 145, 161, 1000, 2049, 0)),
    "mlp0": W.WORKLOADS["long128k_b10"].replace(name="mlp_small", batch=2, ctx=3000, budget_permille=0),
    "mlp100": W.WORKLOADS["long128k_b10"].replace(name="mlp_small", batch=2, ctx=3000, budget_permille=100),
    "mlp500": W.WORKLOADS["long128k_b10"].replace(name="mlp_small", batch=2, ctx=3000, budget_permille=500),
    "mlp1000": W.WORKLOADS["long128k_b10"].replace(name="mlp_small", batch=2, ctx=3000,
                                                   budget_permille=1000),
    "mha_f32": W.Workload("mha", 2, 8, 8, 128, ctx=700, src_dtype="f32", mask="bernoulli"),
    "gqa2_d64": W.Workload("gqa2", 3, 4, 2, 64, ctx_list=(300, 1000, 2500), mask="mlp",
                           budget_permille=400),
    "kv4_mlp": W.WORKLOADS["long128k_kv4_b10"].replace(name="kv4_small", batch=3, ctx=None,
                                                       ctx_list=(1, 40, 2000), budget_permille=300),
    "kv4_bern_f32": W.Workload("kv4b", 2, 4, 4, 64, ctx_list=(33, 900), src_dtype="f32",
                               mask="bernoulli", protect=False),
}


@pytest.mark.parametrize("name", sorted(SMALL))
def test_pool_small_every_pair(name):
    check_workload(SMALL[name], pool=True)


def test_pool_tail_holds_garbage():
    """Slots past each pool's count (read by the last, partial tile of a chunk)
    may hold anything: NaN-filled tails change nothing."""
    w = SMALL["mlp500"].replace(name="tailjunk", ctx_list=(1013, 2979), ctx=None)
    lc = LayerCache(w, pool=True)
    q = lc.queries(0)
    _, out0, lse0 = run_attention(lc, q=q)
    hdr = lc.cache.pool_header.cpu().numpy()
    pool = lc.cache.pool.view(w.batch, w.kv_heads, -1)
    for b in range(w.batch):
        for h in range(w.kv_heads):
            n = int(hdr[b, h, 0])
            nt = (n + 31) // 32
            pool[b, h, nt * 40 * w.head_dim:] = 0xFF
            # and the unused records of the last partial tile
            t = n % 32
            if t:
                tile = pool[b, h, (nt - 1) * 40 * w.head_dim: nt * 40 * w.head_dim]
                junk = torch.full_like(tile, 0xFF)
                # keep the used records: rewrite them from a copy of the tile after the fill
                keep = tile.clone()
                tile.copy_(junk)
                _restore_records(tile, keep, t, w.head_dim)
    qn, out1, lse1 = run_attention(lc, q=q)
    assert np.isfinite(out1).all()
    np.testing.assert_array_equal(out1, out0)
    np.testing.assert_array_equal(lse1, lse0)


def _restore_records(tile, keep, t, D):
    """Copy back the bytes of records [0, t) of a tile (per the tile layout)."""
    import numpy as np  # noqa: F811

    k = keep.cpu().numpy()
    cur = tile.cpu().numpy()
    NG, SB, VD = D // 32, D // 8, D // 8
    for r in range(t):
        row, j = ((r >> 4) << 2) + ((r & 15) >> 2), r & 3
        for s in range(4):
            o = ((r >> 4) * 64 + s * 16 + (r & 15)) * SB
            cur[o:o + SB] = k[o:o + SB]
        for g in range(NG):
            for base in (16 * D, 36 * D):
                o = base + ((row * NG + g) * 4 + j) * 4
                cur[o:o + 4] = k[o:o + 4]
        for d in range(VD):
            o = 20 * D + ((row * VD + d) * 4 + j) * 4
            cur[o:o + 4] = k[o:o + 4]
    tile.copy_(torch.from_numpy(cur))


def _pool_decode_run(w, steps, budgets, stall=(), shrink=None, attend_every=25, fused_reappend=False):
    """Decode steps with the refresh state on a pooled cache: after every step the
    mask equals the oracle's top-k of the GPU's own scores and the pool holds exactly
    the kept records; attention is checked against the oracle every few steps.
    ``shrink`` = (step, b, by): at that step sequence b is rolled back by `by`
    positions and its recent window appended again (the rollback contract), with
    kvc_quantize_append or, with ``fused_reappend``, the fused append + refresh."""
    m = kvc()
    lc = LayerCache(w, pool=True, errors=True)
    state = m.topk_workspace(lc.cache)
    lens = lc.lengths.copy()
    ns, nr = prot(w)
    for step in range(steps):
        budget = budgets(step)
        n_new = np.ones(w.batch, np.int32)
        for (s, b) in stall:
            if s == step:
                n_new[b] = 0
        if shrink is not None and shrink[0] == step:
            _, b0, by = shrink
            # roll sequence b0 back, then append its recent window again
            lens[b0] -= by
            n_re = min(nr, int(lens[b0]) - ns) if w.protect else 0
            n_new[b0] = 0
            lc.seq_lens.copy_(torch.from_numpy(lens.astype(np.int32)))
            if n_re > 0:
                L0 = int(lens[b0])
                rows_k = torch.zeros((w.batch, n_re, w.kv_heads, w.head_dim), dtype=torch.bfloat16,
                                     device="cuda")
                rows_v = torch.zeros_like(rows_k)
                rows_k[b0] = W.kv_source_torch(w, 0, "K", b0, L0 - n_re, L0, "cuda")
                rows_v[b0] = W.kv_source_torch(w, 0, "V", b0, L0 - n_re, L0, "cuda")
                nn = torch.zeros(w.batch, dtype=torch.int32, device="cuda")
                nn[b0] = n_re
                if fused_reappend:
                    m.kvc_append_score_topk_mask(lc.cache, lc.mlp, rows_k, rows_v, nn, budget, ws=state)
                else:
                    m.kvc_quantize_append(lc.cache, rows_k, rows_v, nn)
        k_new = W.kv_rows_torch(w, 0, "K", lens, "cuda")[:, None]
        v_new = W.kv_rows_torch(w, 0, "V", lens, "cuda")[:, None]
        lens += n_new
        lc.seq_lens.copy_(torch.from_numpy(lens.astype(np.int32)))
        lc.lengths = lens.copy()
        nn = torch.from_numpy(n_new).cuda()
        if w.mask != "mlp":
            # caller-written scores: write those of the appended positions, then
            # refresh with n_new (the older scores are declared unchanged)
            # (odd steps: the two in one call, which runs as one launch)
            if not (step % 2 and w.protect):
                m.kvc_quantize_append(lc.cache, k_new, v_new, nn)
            if w.mask == "scores":
                for b in range(w.batch):
                    if n_new[b]:
                        L = int(lens[b])
                        lc.cache.scores[b, :, L - 1] = W.given_scores_torch(w, 0, b, L, "cuda")[:, L - 1]
            if step % 2 and w.protect:
                m.kvc_append_score_topk_mask(lc.cache, None, k_new, v_new, nn, budget, ws=state)
            else:
                m.kvc_score_topk_mask(lc.cache, None, None, None, nn, budget, ws=state)
        elif step % 2 and w.protect:
            m.kvc_append_score_topk_mask(lc.cache, lc.mlp, k_new, v_new, nn, budget, ws=state)
        else:
            m.kvc_quantize_append(lc.cache, k_new, v_new, nn)
            m.kvc_score_topk_mask(lc.cache, lc.mlp, k_new, v_new, nn, budget, ws=state)
        cpu = cpu_buffers(lc)
        for b in range(w.batch):
            L = int(lens[b])
            start, n4 = regions.int4_range(L, ns, nr)
            for h in range(w.kv_heads):
                bits = mask_bits(cpu["keep_mask"][b, h], cpu["keep_mask"].shape[-1] * 32)
                want = policy.topk_keep(cpu["scores"][b, h, start:start + n4].astype(np.float64), budget)
                assert np.array_equal(bits[start:start + n4], want), f"step {step} b={b} h={h}"
                check_pool(cpu, b, h, L, bits[start:start + n4], w.head_dim, ns)
        if step % attend_every == attend_every - 1 or (shrink is not None and step == shrink[0]):
            qn, out, lse = run_attention(lc, step=step)
            G = w.group_size
            for b in range(w.batch):
                L = int(lens[b])
                for h in range(w.kv_heads):
                    keep4 = keep4_from_mask(cpu["keep_mask"][b, h], L, ns, nr)
                    ro, rl = oracle_heads(w, 0, b, h, L, keep4, qn[b, h * G:(h + 1) * G])
                    assert_attention_close(out[b, h * G:(h + 1) * G], lse[b, h * G:(h + 1) * G], ro, rl,
                                           f"step {step} b={b} h={h}")
    assert lc.cache.error_bits() == 0
    return lc


def test_pool_incremental_every_step():
    """400 steps: lists drain and rebuild (full refreshes update the pool from the
    changed mask bits), a budget change at step 300, stalled sequences; pool checked
    every step."""
    w = W.WORKLOADS["fullstep"].replace(name="pinc", batch=3, kv_heads=2, q_heads=8, layers=1,
                                        ctx=2000, ctx_list=(140, 700, 2000), decode_steps=400,
                                        budget_permille=500)  # the pool holds the larger budget
    _pool_decode_run(w, 400, lambda s: 500 if s < 300 else 300, stall=[(50, 1), (51, 1), (120, 2)])


def test_pool_pure_kv4_incremental():
    w = W.WORKLOADS["long128k_kv4_b10"].replace(name="pkv4", batch=2, kv_heads=2, q_heads=4,
                                                ctx=None, ctx_list=(3, 1200), decode_steps=120,
                                                budget_permille=400)
    _pool_decode_run(w, 120, lambda s: 400)


def test_pool_given_scores_incremental():
    """Caller-written scores (the long-tail workload's kind) with n_new declaring
    the older scores unchanged: the refresh state's in-place update runs without
    an MLP; mask and pool checked every step across the recent window's edge."""
    w = W.WORKLOADS["longtail"].replace(name="given_inc", batch=4, kv_heads=2, q_heads=8,
                                        ctx_range=None, ctx_list=(150, 400, 1500, 3000),
                                        decode_steps=200)
    _pool_decode_run(w, 160, lambda s: 500 if s < 100 else 400, stall=[(30, 2)], attend_every=40)


def test_pool_decode_steps_many_pairs():
    """600 pairs: a decode step packs five pairs per refresh workgroup (one wave
    each), and the budget change at step 5 makes every pair's step fall back to
    the full refresh, the pairs of a workgroup taking turns. Masks and pools
    match the oracle after every step."""
    lens = tuple(int(x) for x in np.linspace(150, 600, 150).round())
    w = W.WORKLOADS["longtail"].replace(name="many_steps", batch=len(lens), kv_heads=4, q_heads=16,
                                        ctx_range=None, ctx_list=lens, decode_steps=12)
    _pool_decode_run(w, 10, lambda s: 500 if s < 5 else 400, attend_every=100)


def test_pool_decode_steps_sixteen_pairs_per_workgroup():
    """2,048 pairs: a decode step packs sixteen pairs per refresh workgroup (one
    wave each), and the budget change at step 3 makes all sixteen of a
    workgroup's pairs fall back to the full refresh in turn. Masks and pools
    match the oracle after every step."""
    lens = tuple(int(x) for x in np.linspace(150, 420, 256).round())
    w = W.WORKLOADS["longtail"].replace(name="sixteen_steps", batch=len(lens), kv_heads=8, q_heads=32,
                                        ctx_range=None, ctx_list=lens, decode_steps=8)
    _pool_decode_run(w, 6, lambda s: 500 if s < 3 else 400, attend_every=100)


def test_pool_keep_all_incremental():
    """Every position kept (budget 1000, the uniform workload's mask) refreshed in
    place each step: each record entering the INT4 region joins the pool."""
    w = W.WORKLOADS["uniform4k"].replace(name="all_inc", batch=3, kv_heads=2, q_heads=8,
                                         ctx=None, ctx_list=(100, 700, 2000), decode_steps=160)
    _pool_decode_run(w, 150, lambda s: 1000, attend_every=50)


def test_rollback_reappend_restores_parity():
    """A sequence rolled back by 37 positions and its recent window appended
    again: mask, pool and attention match the oracle at the shorter length."""
    w = W.WORKLOADS["fullstep"].replace(name="rollback", batch=2, kv_heads=2, q_heads=8, layers=1,
                                        ctx=900, ctx_list=(600, 900), decode_steps=80)
    _pool_decode_run(w, 60, lambda s: 300, shrink=(40, 1, 37), attend_every=20)


def test_rollback_fused_reappend():
    """The same rollback with the recent window appended again by the fused append +
    score + refresh call: the pool is updated from the changed mask bits (the
    rewritten rows sit outside the INT4 region at the shorter length)."""
    w = W.WORKLOADS["fullstep"].replace(name="rollback_f", batch=2, kv_heads=2, q_heads=8, layers=1,
                                        ctx=900, ctx_list=(600, 900), decode_steps=80)
    _pool_decode_run(w, 60, lambda s: 300, shrink=(40, 1, 37), attend_every=20, fused_reappend=True)


def test_pool_budget_swings():
    """Full refreshes that grow the kept set (entering records fill the slots of
    leaving ones, then extend the pool), shrink it (tail records move into holes),
    empty it, and change it by more than 1024 records (rebuilt); checked every step."""
    w = W.WORKLOADS["fullstep"].replace(name="swing", batch=2, kv_heads=2, q_heads=8, layers=1,
                                        ctx=None, ctx_list=(3000, 9000), decode_steps=14,
                                        budget_permille=600)
    sched = [600, 600, 300, 300, 500, 100, 100, 600, 450, 450, 0, 0, 600, 590]
    _pool_decode_run(w, len(sched), lambda s: sched[s], attend_every=4)


def test_pool_sequence_written_afresh():
    """A sequence written afresh over its pages (other rows, a shorter length) and
    refreshed: the append clears the pool's validity word, the refresh rebuilds the
    pool, and pool and attention match the oracle on the new rows."""
    m = kvc()
    w = SMALL["mlp500"].replace(name="afresh", batch=2, ctx=None, ctx_list=(1500, 2500))
    lc = LayerCache(w, pool=True, errors=True)
    c = lc.cache
    state = m.topk_workspace(c)
    m.kvc_score_topk_mask(c, None, None, None, None, w.budget_permille, ws=state)
    L1 = 2000
    lens = lc.lengths.copy()
    lens[1] = L1
    lc.seq_lens.copy_(torch.from_numpy(lens.astype(np.int32)))
    lc.lengths = lens.copy()
    dt = torch.bfloat16 if w.src_dtype == "bf16" else torch.float32
    rows_k = torch.zeros((w.batch, L1, w.kv_heads, w.head_dim), dtype=dt, device="cuda")
    rows_v = torch.zeros_like(rows_k)
    rows_k[1] = W.kv_source_torch(w, 1, "K", 1, 0, L1, "cuda")  # layer 1's rows: other contents
    rows_v[1] = W.kv_source_torch(w, 1, "V", 1, 0, L1, "cuda")
    nn = torch.tensor([0, L1], dtype=torch.int32, device="cuda")
    m.kvc_quantize_append(c, rows_k, rows_v, nn)
    torch.cuda.synchronize()
    assert (c.pool_header[1, :, 2] == 0).all(), "the rewrite did not clear the pool's validity word"
    assert (c.pool_header[0, :, 2] != 0).all()
    m.kvc_score_topk_mask(c, lc.mlp, rows_k, rows_v, nn, w.budget_permille, ws=state)
    cpu = cpu_buffers(lc)
    ns, nr = prot(w)
    qn, out, lse = run_attention(lc, step=3)
    G = w.group_size
    for b, layer in ((0, 0), (1, 1)):
        L = int(lens[b])
        start, n4 = regions.int4_range(L, ns, nr)
        for h in range(w.kv_heads):
            bits = mask_bits(cpu["keep_mask"][b, h], cpu["keep_mask"].shape[-1] * 32)
            want = policy.topk_keep(cpu["scores"][b, h, start:start + n4].astype(np.float64),
                                    w.budget_permille)
            assert np.array_equal(bits[start:start + n4], want), f"b={b} h={h}"
            check_pool(cpu, b, h, L, bits[start:start + n4], w.head_dim, ns)
            keep4 = keep4_from_mask(cpu["keep_mask"][b, h], L, ns, nr)
            ro, rl = oracle_heads(w, layer, b, h, L, keep4, qn[b, h * G:(h + 1) * G])
            assert_attention_close(out[b, h * G:(h + 1) * G], lse[b, h * G:(h + 1) * G], ro, rl,
                                   f"afresh b={b} h={h}")
    assert c.error_bits() == 0


@pytest.mark.parametrize("name", ["long128k_b10", "long128k_b50", "uniform4k", "longtail"])
def test_pool_full_size_sampled(name):
    w = W.WORKLOADS[name]
    pairs = [(0, 0), (3, 7), (1, 4)] if w.batch == 4 else sample_pairs(w, 3, 5)
    if name == "longtail":
        lens = w.lengths()
        pairs += [(int(np.argmax(lens)), 7), (int(np.argmin(lens)), 0)]
    check_workload(w, pairs, pool=True)


def test_pool_full_decode_step_layer_sampled():
    """One layer of the 36-layer workload in pool mode: prefill, one fused decode step."""
    m = kvc()
    w = W.WORKLOADS["fullstep"]
    lc = LayerCache(w, keep_sources=False, pool=True)
    state = m.topk_workspace(lc.cache)
    m.kvc_score_topk_mask(lc.cache, None, None, None, None, w.budget_permille, ws=state)
    lens = lc.lengths.copy()
    k_new = W.kv_rows_torch(w, 0, "K", lens, "cuda")[:, None]
    v_new = W.kv_rows_torch(w, 0, "V", lens, "cuda")[:, None]
    lens += 1
    lc.seq_lens.copy_(torch.from_numpy(lens.astype(np.int32)))
    lc.lengths = lens.copy()
    one = torch.ones(w.batch, dtype=torch.int32, device="cuda")
    m.kvc_append_score_topk_mask(lc.cache, lc.mlp, k_new, v_new, one, w.budget_permille, ws=state)
    from test_gpu_parity import check_pair

    cpu = cpu_buffers(lc)
    qn, out, lse = run_attention(lc, step=1)
    for b, h in [(0, 0), (77, 5), (127, 7)]:
        print(f"  check fullstep pool b={b} kvh={h}", flush=True)
        check_pair(w, lc, cpu, qn, out, lse, b, h)


def test_pool_and_mask_modes_agree_and_rerun_is_bit_identical():
    w = SMALL["mlp500"].replace(name="modes", batch=3, ctx=None, ctx_list=(145, 1999, 3000))
    lc = LayerCache(w, pool=True)
    q = lc.queries(0)
    _, o_pool, l_pool = run_attention(lc, q=q)
    _, o_pool2, l_pool2 = run_attention(lc, q=q)
    np.testing.assert_array_equal(o_pool, o_pool2)
    np.testing.assert_array_equal(l_pool, l_pool2)
    # the same cache through the mask (a descriptor copy without the pool)
    import copy

    c = lc.cache
    masked = copy.copy(c)
    masked.desc = type(c.desc).from_buffer_copy(c.desc)
    masked.desc.pool_capacity = 0
    out = torch.empty((w.batch, w.q_heads, w.head_dim), dtype=torch.float32, device="cuda")
    lse = torch.empty((w.batch, w.q_heads), dtype=torch.float32, device="cuda")
    kvc().kvc_decode_attention(masked, q, out, lse, lc.workspace())
    torch.cuda.synchronize()
    assert np.abs(out.cpu().numpy() - o_pool).max() < 1e-4
    assert np.abs(lse.cpu().numpy() - l_pool).max() < 1e-4


def test_pool_one_chunk_per_pair_many_pairs_rerun_is_bit_identical():
    """More pairs than the 512 resident chunk workgroups, one chunk per pair:
    separate INT8 workgroups run after the chunks, and one that finds its
    chunk already counted merges from LDS without storing its own partial
    (else it stores it and the last of the two merges). Either way the output
    is the same bits: five calls are bit-identical, and sampled pairs (the
    shortest, the longest and others) match the oracle."""
    lens = tuple(int(x) for x in np.linspace(145, 1000, 72).round()[::-1])
    w = W.WORKLOADS["longtail"].replace(name="many_pairs", batch=len(lens), ctx_range=None,
                                        ctx_list=lens)
    lc = check_workload(w, [(0, 0), (71, 7), (35, 3), (10, 5), (60, 1)], pool=True)
    q = lc.queries(0)
    _, o0, l0 = run_attention(lc, q=q)
    for _ in range(4):
        _, o1, l1 = run_attention(lc, q=q)
        np.testing.assert_array_equal(o0, o1)
        np.testing.assert_array_equal(l0, l1)


def test_error_word():
    """Lengths beyond max_ctx, table entries outside the pools and a pool that no
    longer describes the length set their bits; a clean run sets none."""
    m = kvc()
    w = SMALL["mlp500"].replace(name="errs", batch=2, ctx=None, ctx_list=(1500, 2500), decode_steps=4)
    lc = LayerCache(w, pool=True, errors=True)
    c = lc.cache
    run_attention(lc)
    assert c.error_bits() == 0
    # an append without a refresh: the pool describes the previous length
    lens = lc.lengths.copy()
    k_new = W.kv_rows_torch(w, 0, "K", lens, "cuda")[:, None]
    v_new = W.kv_rows_torch(w, 0, "V", lens, "cuda")[:, None]
    lens += 1
    lc.seq_lens.copy_(torch.from_numpy(lens.astype(np.int32)))
    m.kvc_quantize_append(c, k_new, v_new, torch.ones(w.batch, dtype=torch.int32, device="cuda"))
    run_attention(lc)
    assert c.error_bits() & m.KVC_ERR_POOL
    c.errors.zero_()
    # a refresh brings the pool up to date
    m.kvc_score_topk_mask(c, None, None, None, None, w.budget_permille)
    run_attention(lc)
    assert c.error_bits() == 0
    # a table entry outside the page pools, inside the INT4 region
    saved = lc.table[1, 20].item()
    lc.table[1, 20] = 1 << 30
    m.kvc_score_topk_mask(c, None, None, None, None, w.budget_permille)
    torch.cuda.synchronize()
    assert c.error_bits() & m.KVC_ERR_PAGE
    lc.table[1, 20] = saved
    c.errors.zero_()
    # a length beyond max_ctx
    lc.seq_lens[0] = lc.max_ctx + 5
    run_attention(lc)
    assert c.error_bits() & m.KVC_ERR_LENGTH
    lc.seq_lens[0] = int(lens[0])


def _block_pool_run(w, steps, plan, stall=(), attend_every=20):
    """Decode steps of the block policy on a pooled cache through one block
    refresh state (even steps: append, then kvc_score_block_mask; odd steps: the
    fused kvc_append_score_block_mask): after every step the mask equals the
    oracle's block policy on the GPU's scores and the pool holds exactly the kept
    records; attention over the pool is checked against the oracle every few steps."""
    m = kvc()
    lc = LayerCache(w, pool=True, errors=True)
    state = m.block_workspace(lc.cache, 16)  # the largest of the three sizes
    lens = lc.lengths.copy()
    ns, nr = prot(w)
    for step in range(steps):
        budget, window, block = plan(step)
        n_new = np.ones(w.batch, np.int32)
        for (s_, b) in stall:
            if s_ == step:
                n_new[b] = 0
        k_new = W.kv_rows_torch(w, 0, "K", lens, "cuda")[:, None]
        v_new = W.kv_rows_torch(w, 0, "V", lens, "cuda")[:, None]
        lens += n_new
        lc.seq_lens.copy_(torch.from_numpy(lens.astype(np.int32)))
        lc.lengths = lens.copy()
        nn = torch.from_numpy(n_new).cuda()
        if step % 2:
            m.kvc_append_score_block_mask(lc.cache, lc.mlp, k_new, v_new, nn, budget, window, block,
                                          ws=state)
        else:
            m.kvc_quantize_append(lc.cache, k_new, v_new, nn)
            m.kvc_score_block_mask(lc.cache, lc.mlp, k_new, v_new, nn, budget, window, block, ws=state)
        cpu = cpu_buffers(lc)
        for b in range(w.batch):
            L = int(lens[b])
            start, n4 = regions.int4_range(L, ns, nr)
            for h in range(w.kv_heads):
                bits = mask_bits(cpu["keep_mask"][b, h], cpu["keep_mask"].shape[-1] * 32)
                want = policy.block_keep(cpu["scores"][b, h, start:start + n4], budget, block, window)
                assert np.array_equal(bits[start:start + n4], want), f"step {step} b={b} h={h}"
                check_pool(cpu, b, h, L, bits[start:start + n4], w.head_dim, ns)
        if step % attend_every == attend_every - 1:
            qn, out, lse = run_attention(lc, step=step)
            G = w.group_size
            for b in range(w.batch):
                L = int(lens[b])
                for h in range(w.kv_heads):
                    keep4 = keep4_from_mask(cpu["keep_mask"][b, h], L, ns, nr)
                    ro, rl = oracle_heads(w, 0, b, h, L, keep4, qn[b, h * G:(h + 1) * G])
                    assert_attention_close(out[b, h * G:(h + 1) * G], lse[b, h * G:(h + 1) * G], ro, rl,
                                           f"step {step} b={b} h={h}")
    assert lc.cache.error_bits() == 0
    return lc


def test_block_pool_every_step():
    """The block policy maintains the pool too: 240 steps through one state while
    the budget changes (the threshold moves by many blocks: records move in place),
    sequences stall, and the window and the block size change (state and, where
    more than 1024 records change, the pool rebuilt); pool checked every step."""
    w = W.WORKLOADS["fullstep"].replace(name="blk_pool", batch=3, kv_heads=2, q_heads=8, layers=1,
                                        ctx=2500, ctx_list=(140, 700, 2500), decode_steps=240,
                                        policy="block", budget_permille=400)

    def plan(step):
        budget = 300 if step < 60 else 120
        window = 0 if step < 120 else 600
        block = 16 if step < 160 else (32 if step < 200 else 64)
        return budget, window, block

    _block_pool_run(w, 240, plan, stall=[(40, 0), (41, 0), (100, 2)])


def test_block_pool_pure_kv4_d64():
    """The block policy's pool without INT8 protection (every appended position
    is a candidate at once) at D = 64 (two pool tiles per ring slot), with
    32-token blocks: pool and mask checked every step."""
    w = W.Workload("blk_pool_kv4", 3, 8, 2, 64, ctx_list=(40, 700, 1900), mask="mlp",
                   budget_permille=400, policy="block", block_tokens=32, protect=False,
                   decode_steps=80)
    _block_pool_run(w, 70, lambda s: (300 if s < 35 else 150, 0, 32), stall=[(20, 1)], attend_every=14)


def test_block_pool_full_size_sampled():
    """The 128K block workloads with a pool: a few decode steps, then attention
    over the pool on sampled pairs against the oracle, and against attention
    through the mask on the same cache (reads the same records)."""
    import decode_attention_compressed_quantize_amd as m

    for name in ("long128k_blk_b10", "long128k_blk_b50"):
        w = W.WORKLOADS[name].replace(decode_steps=8)  # room for the appended positions
        lc = LayerCache(w, pool=True, errors=True)
        state = m.block_workspace(lc.cache, w.block_tokens)
        lens = lc.lengths.copy()
        for step in range(3):
            k_new = W.kv_rows_torch(w, 0, "K", lens, "cuda")[:, None]
            v_new = W.kv_rows_torch(w, 0, "V", lens, "cuda")[:, None]
            lens += 1
            lc.seq_lens.copy_(torch.from_numpy(lens.astype(np.int32)))
            lc.lengths = lens.copy()
            nn = torch.ones(w.batch, dtype=torch.int32, device="cuda")
            m.kvc_append_score_block_mask(lc.cache, lc.mlp, k_new, v_new, nn, w.budget_permille,
                                          w.recency_window, w.block_tokens, ws=state)
        print(f"{name}: errors {lc.cache.error_bits()} headers "
              f"{lc.cache.pool_header[:, :, :3].cpu().numpy().reshape(-1, 3)[:8].tolist()}", flush=True)
        cpu = cpu_buffers(lc)
        ns, nr = prot(w)
        for (b, h) in sample_pairs(w, 4, 7):
            L = int(lens[b])
            start, n4 = regions.int4_range(L, ns, nr)
            bits = mask_bits(cpu["keep_mask"][b, h], cpu["keep_mask"].shape[-1] * 32)
            check_pool(cpu, b, h, L, bits[start:start + n4], w.head_dim, ns)
        qn, out, lse = run_attention(lc, step=3)
        mask = cpu["keep_mask"]
        G = w.group_size
        for (b, h) in sample_pairs(w, 4, 7):
            L = int(lens[b])
            keep4 = keep4_from_mask(mask[b, h], L)
            ro, rl = oracle_heads(w, 0, b, h, L, keep4, qn[b, h * G:(h + 1) * G])
            assert_attention_close(out[b, h * G:(h + 1) * G], lse[b, h * G:(h + 1) * G], ro, rl,
                                   f"{name} b={b} h={h}")
        assert lc.cache.error_bits() == 0
        print(f"{name}: pool counts {lc.cache.pool_header[:, :, 0].flatten().tolist()[:4]}...", flush=True)
        del lc
