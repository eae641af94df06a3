"""GPU parity of the learner-side shadow-mask attention against the oracle.

Rows come either from random bits or from rollouts recorded on the GPU (the
decode path's keep masks after every step, under the token, block and pure
KV4 policies). Outputs within max-abs 2e-3 and rel-L2 1e-3, LSE within 2e-3
of the float64 oracle; rows that attend nothing must give 0 and -inf.
"""
import numpy as np
import pytest

import workloads as W
from kvc_testlib import assert_attention_close, mask_bits, to_f32
from oracle import shadow as oshadow

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _needs_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def kvc():
    import decode_attention_compressed_quantize_amd as m

    return m


def learner_inputs(w, lens, T):
    """bf16 q [B][T][Hq][D], k, v [B][T][Hkv][D] from the workload's sources."""
    B = len(lens)
    q = torch.zeros((B, T, w.q_heads, w.head_dim), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((B, T, w.kv_heads, w.head_dim), dtype=torch.bfloat16, device="cuda")
    v = torch.zeros_like(k)
    for b, L in enumerate(lens):
        L = int(L)
        if L == 0:
            continue
        q[b, :L] = W.learner_queries_torch(w, 0, b, 0, L, "cuda")
        k[b, :L] = W.kv_source_torch(w, 0, "K", b, 0, L, "cuda")
        v[b, :L] = W.kv_source_torch(w, 0, "V", b, 0, L, "cuda")
    return q, k, v


def packed_rows(dense):
    """bool [..][n*32] -> int32 words on the GPU (bit t%32 of word t/32)."""
    packed = np.packbits(dense, axis=-1, bitorder="little").view(np.uint32)
    return torch.from_numpy(packed.view(np.int32).copy()).cuda()


def run(q, k, v, lens, prompts, rows):
    B, T, Hq, D = q.shape
    out = torch.full((B, T, Hq, D), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((B, T, Hq), float("nan"), dtype=torch.float32, device="cuda")
    sl = torch.tensor(np.asarray(lens, np.int32), device="cuda")
    pl = torch.tensor(np.asarray(prompts, np.int32), device="cuda")
    kvc().kvc_shadow_attention(q, k, v, sl, pl, rows, out, lse)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy()


def bits_of(rows_np, T):
    """int32 words [..][words] -> bool [..][T] (bit t%32 of word t/32)."""
    b = np.unpackbits(np.ascontiguousarray(rows_np).view(np.uint8), axis=-1, bitorder="little")
    return b[..., :T].astype(bool)


def check(w, q, k, v, lens, prompts, rows, out, lse, sample=None, seed=0):
    qn = to_f32(q.cpu().view(torch.int16).numpy().view(np.uint16))
    kn = to_f32(k.cpu().view(torch.int16).numpy().view(np.uint16))
    vn = to_f32(v.cpu().view(torch.int16).numpy().view(np.uint16))
    T = q.shape[1]
    rb = bits_of(rows.cpu().numpy(), T) if rows is not None else None
    rng = np.random.default_rng(seed)
    for b, L in enumerate(lens):
        L, P = int(L), int(prompts[b])
        if L == 0:
            continue
        nrows = rb.shape[2] if rb is not None else 0
        srows = np.zeros((max(0, L - P), w.kv_heads, T), bool)
        n = min(nrows, L - P)
        if n > 0:
            srows[:n] = np.transpose(rb[b, :, :n], (1, 0, 2))
        if sample is None:
            ro, rl = oshadow.shadow_attention(qn[b, :L], kn[b, :L], vn[b, :L], P, srows)
            picks = range(L)
        else:
            picks = sorted(set(rng.integers(0, L, sample).tolist()) | {0, L - 1, min(P, L - 1)})
            ro = np.zeros((L, w.q_heads, w.head_dim))
            rl = np.zeros((L, w.q_heads))
            G = w.q_heads // w.kv_heads
            from oracle import attention
            for p in picks:
                for g in range(w.kv_heads):
                    pos = oshadow.allowed_positions(p, P, srows[p - P, g] if p >= P else None)
                    hs = slice(g * G, (g + 1) * G)
                    ro[p, hs], rl[p, hs] = attention.attend(qn[b, p, hs].astype(np.float64),
                                                            kn[b, pos, g].astype(np.float64),
                                                            vn[b, pos, g].astype(np.float64))
        picks = list(picks)
        err = assert_attention_close(out[b, picks], lse[b, picks], ro[picks], rl[picks],
                                     what=f"{w.name} b={b}")
        print(f"  {w.name} b={b} L={L} P={P}: rows {len(picks)} max-abs {err[0]:.2e} "
              f"rel-L2 {err[1]:.2e} lse {err[2]:.2e}", flush=True)
        assert np.isnan(out[b, L:]).all(), "rows at and beyond L must not be written"


@pytest.mark.parametrize("Hq,Hkv,D", [(8, 2, 128), (4, 2, 128), (2, 2, 64), (8, 2, 64)])
def test_random_rows_every_position(Hq, Hkv, D):
    w = W.Workload(f"sa_rand_{Hq}_{Hkv}_{D}", 3, Hq, Hkv, D)
    lens, prompts, T = (300, 517, 70), (100, 0, 70), 523
    q, k, v = learner_inputs(w, lens, T)
    rng = np.random.default_rng(Hq * 100 + D)
    words = (T + 31) // 32
    dense = rng.random((3, Hkv, 517, words * 32)) < 0.3
    dense[:, :, 7] = False  # a row that attends nothing
    rows = packed_rows(dense)
    out, lse = run(q, k, v, lens, prompts, rows)
    check(w, q, k, v, lens, prompts, rows, out, lse)


def test_edges_no_generated_rows_length_one_and_missing_rows():
    w = W.Workload("sa_edges", 4, 8, 2, 128)
    lens, prompts, T = (1, 40, 200, 0), (0, 40, 150, 0), 201
    q, k, v = learner_inputs(w, lens, T)
    words = (T + 31) // 32
    rows = torch.full((4, 2, 20, words), -1, dtype=torch.int32, device="cuda")  # 20 rows only
    out, lse = run(q, k, v, lens, prompts, rows)
    check(w, q, k, v, lens, prompts, rows, out, lse)
    # sequence 2: generated positions 170..199 have no row and attend nothing
    assert np.all(out[2, 170:200] == 0.0) and np.all(np.isneginf(lse[2, 170:200]))
    out0, lse0 = run(q, k, v, lens, prompts, None)  # no record at all
    assert np.all(out0[2, 150:200] == 0.0)


def recorded(w, steps):
    from decode_attention_compressed_quantize_amd.workload_cache import LayerCache

    lc = LayerCache(w.replace(decode_steps=steps), keep_sources=False)
    prompts = lc.lengths.copy()
    rows, lens = lc.record_rollout(steps, ws=lc.refresh_state())
    return lc, prompts, rows, lens


@pytest.mark.parametrize("policy,protect", [("token", True), ("block", True), ("token", False)])
def test_recorded_rollout_rows(policy, protect):
    """Rows recorded from GPU decode steps (append, score, refresh) drive the
    learner's attention; every generated row and a sample of prompt rows."""
    w = W.Workload(f"sa_roll_{policy}_{int(protect)}", 2, 8, 2, 128, ctx_list=(600, 333),
                   mask="mlp", budget_permille=300, policy=policy, protect=protect)
    lc, prompts, rows, lens = recorded(w, 150)
    T = int(lens.max())
    q, k, v = learner_inputs(w, lens, T)
    out, lse = run(q, k, v, lens, prompts, rows)
    check(w, q, k, v, lens, prompts, rows, out, lse)


def test_long_sequence_sampled_rows():
    """8K positions (4K prompt, 4K generated rows at 30% kept), 32 query / 8 kv heads."""
    T, P = 8192, 4096
    w = W.Workload("sa_long", 1, 32, 8, 128, ctx=T)
    q, k, v = learner_inputs(w, (T,), T)
    rng = np.random.default_rng(5)
    rows = packed_rows(rng.integers(0, 10, (1, 8, T - P, T), dtype=np.uint8) < 3)
    out, lse = run(q, k, v, (T,), (P,), rows)
    check(w, q, k, v, (T,), (P,), rows, out, lse, sample=24, seed=1)
