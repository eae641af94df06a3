"""GPU tests of the host tier: INT4 pages in pinned host memory.

Attention and the append read and write pages of either tier in place, so a
cache whose pages were moved between tiers must give bit-identical attention;
page lists and copies are checked against numpy, and decode steps that append
into host pages against the oracle.
"""
import numpy as np
import pytest

import workloads as W
from kvc_testlib import mask_bits, prot
from oracle import regions

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _needs_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def kvc():
    import decode_attention_compressed_quantize_amd as m

    return m


def make(w, host_pages=None):
    """A cache with a host tier as large as its device pool (or ``host_pages``)."""
    from decode_attention_compressed_quantize_amd.workload_cache import LayerCache

    _, num_pages = W.page_table(w, 0)
    return LayerCache(w, host_pages=num_pages if host_pages is None else host_pages)


def attend(lc, q):
    w = lc.w
    out = torch.empty((w.batch, w.q_heads, w.head_dim), dtype=torch.float32, device="cuda")
    lse = torch.empty((w.batch, w.q_heads), dtype=torch.float32, device="cuda")
    kvc().kvc_decode_attention(lc.cache, q, out, lse, lc.workspace())
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy()


def tier_cpu(lc):
    """CPU copies of the cache with both pools concatenated (page ids index them)."""
    c = lc.cache
    torch.cuda.synchronize()
    return {
        "int4_codes": np.concatenate([c.int4_codes.cpu().numpy(), c.int4_codes_host.numpy()]),
        "int4_meta": np.concatenate([c.int4_meta.cpu().numpy(), c.int4_meta_host.numpy()]),
        "int8_codes": c.int8_codes.cpu().numpy() if c.protect else None,
        "int8_scales": c.int8_scales.cpu().numpy() if c.protect else None,
        "keep_mask": c.keep_mask.cpu().numpy(),
        "scores": c.scores.cpu().numpy(),
        "table": lc.table.cpu().numpy(),
    }


def move_to_host(lc, pairs):
    """Force logical pages (b, lp) onto free host pages."""
    pairs = [(b, lp) for b, lp in pairs if int(lc.table[b, lp]) < lc.num_pages][: len(lc.host_free)]
    if not pairs:
        return 0
    idx = torch.tensor(pairs, dtype=torch.long, device="cuda")
    src = lc.table[idx[:, 0], idx[:, 1]].clone()
    dst = torch.tensor(lc.host_free[: len(pairs)], dtype=torch.int32, device="cuda")
    del lc.host_free[: len(pairs)]
    kvc().kvc_copy_pages(lc.cache, src, dst)
    lc.table[idx[:, 0], idx[:, 1]] = dst
    lc.dev_free.extend(src.tolist())
    return len(pairs)


def expected_pages(lc, mode):
    """numpy reference of kvc_find_pages."""
    w = lc.w
    c = tier_cpu(lc)
    ns, nr = prot(w)
    found = set()
    for b in range(w.batch):
        L = int(lc.lengths[b])
        for lp in range((L + 15) // 16):
            page = int(c["table"][b, lp])
            t0 = 16 * lp
            bits = np.zeros(16, bool)
            for h in range(w.kv_heads):
                bits |= mask_bits(c["keep_mask"][b, h], c["keep_mask"].shape[-1] * 32)[t0:t0 + 16]
            if mode == 0 and page < lc.num_pages and t0 >= ns and t0 + 16 <= L - nr and not bits.any():
                found.add((b, lp))
            if mode == 1 and page >= lc.num_pages and bits.any():
                found.add((b, lp))
    return found


def found_pages(lc, mode):
    cap = lc.w.batch * lc.table.shape[1]
    out = torch.empty((cap, 2), dtype=torch.int32, device="cuda")
    count = torch.empty(1, dtype=torch.int32, device="cuda")
    kvc().kvc_find_pages(lc.cache, mode, out, count)
    n = int(count.item())
    return {(int(b), int(lp)) for b, lp in out[:n].cpu().numpy()}


@pytest.mark.parametrize("policy,protect", [("block", True), ("token", True), ("token", False)])
def test_tiered_attention_is_bit_identical(policy, protect):
    w = W.Workload(f"tier_{policy}_{int(protect)}", 2, 8, 2, 128, ctx_list=(3000, 1700), mask="mlp",
                   budget_permille=100, policy=policy, protect=protect)
    lc = make(w)
    q = lc.queries(0)
    base = attend(lc, q)
    assert found_pages(lc, 0) == expected_pages(lc, 0)
    n_cold = lc.demote_cold_pages()
    assert n_cold > 0
    assert lc.host_resident_pages() == n_cold
    assert found_pages(lc, 0) == set()
    assert np.array_equal(attend(lc, q)[0], base[0]) and np.array_equal(attend(lc, q)[1], base[1])
    # pages with kept tokens streamed from the host tier
    hot = [(b, lp) for b in range(w.batch) for lp in range(2, int(lc.lengths[b]) // 16 - 9, 3)]
    assert move_to_host(lc, hot) > 0
    assert found_pages(lc, 1) == expected_pages(lc, 1) != set()
    got = attend(lc, q)
    assert np.array_equal(got[0], base[0]) and np.array_equal(got[1], base[1])
    # against the oracle through the combined pools
    from test_gpu_parity import check_pair

    qn = q.cpu().view(torch.int16).numpy().view(np.uint16)
    cpu = tier_cpu(lc)
    for b in range(w.batch):
        for h in range(w.kv_heads):
            check_pair(w, lc, cpu, qn, got[0], got[1], b, h)
    n_hot = lc.promote_hot_pages()
    assert n_hot > 0 and found_pages(lc, 1) == set()
    got = attend(lc, q)
    assert np.array_equal(got[0], base[0]) and np.array_equal(got[1], base[1])


def test_copy_pages_round_trip():
    w = W.Workload("tier_copy", 1, 4, 2, 64, ctx=400, mask="all")
    lc = make(w, host_pages=8)
    c = lc.cache
    src = torch.tensor([3, 5, 7], dtype=torch.int32, device="cuda")
    mid = torch.tensor([lc.num_pages + 0, lc.num_pages + 4, lc.num_pages + 7], dtype=torch.int32,
                       device="cuda")
    dst = torch.tensor([0, 1, 2], dtype=torch.int32, device="cuda")
    want_c = c.int4_codes[src.long()].cpu().numpy()
    want_m = c.int4_meta[src.long()].cpu().numpy()
    kvc().kvc_copy_pages(c, src, mid)
    kvc().kvc_copy_pages(c, mid, dst)
    torch.cuda.synchronize()
    assert np.array_equal(c.int4_codes_host[[0, 4, 7]].numpy(), want_c)
    assert np.array_equal(c.int4_meta_host[[0, 4, 7]].numpy(), want_m)
    assert np.array_equal(c.int4_codes[:3].cpu().numpy(), want_c)
    assert np.array_equal(c.int4_meta[:3].cpu().numpy(), want_m)


def test_decode_steps_append_into_host_pages():
    """Each sequence's page that receives the next token lives in the host tier;
    appends, refreshes and attention follow the oracle step by step."""
    from test_gpu_parity import check_pair

    m = kvc()
    w = W.WORKLOADS["fullstep"].replace(name="tier_steps", batch=2, layers=1, ctx=500,
                                        decode_steps=40, ctx_list=(500, 700), kv_heads=2, q_heads=8)
    lc = make(w)
    lens = lc.lengths.copy()
    one = torch.ones(w.batch, dtype=torch.int32, device="cuda")
    state = lc.refresh_state()
    for step in range(1, 41):
        move_to_host(lc, [(b, int(lens[b]) // 16) for b in range(w.batch)])
        k_new = W.kv_rows_torch(w, 0, "K", lens, "cuda")[:, None]
        v_new = W.kv_rows_torch(w, 0, "V", lens, "cuda")[:, None]
        lens += 1
        lc.seq_lens.copy_(torch.from_numpy(lens.astype(np.int32)))
        lc.lengths = lens.copy()
        m.kvc_quantize_append(lc.cache, k_new, v_new, one)
        lc.refresh(k_new, v_new, one, ws=state)
        if step % 10 == 0:
            q = lc.queries(step)
            out, lse = attend(lc, q)
            qn = q.cpu().view(torch.int16).numpy().view(np.uint16)
            cpu = tier_cpu(lc)
            for b in range(w.batch):
                for h in range(w.kv_heads):
                    check_pair(w, lc, cpu, qn, out, lse, b, h)
    assert lc.host_resident_pages() >= 4
