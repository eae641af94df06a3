"""GPU parity of the token-policy top-k refresh on special scores.

The order the refresh implements (score descending, then position ascending;
NaN below every number, -inf included; -0 equal to +0) is checked bit for bit
against ``oracle.policy.topk_keep`` on:

* caller-written scores (``mlp`` NULL: the full radix refresh) holding NaN,
  +-inf, +-0 and long runs of tied values, with and without a refresh state;
* scores the per-head MLP produces on device with weights built so that its
  float32 evaluation overflows to +-inf, cancels to NaN and returns signed
  zeros and ties, through hundreds of decode steps on the refresh state (the
  incremental list update), every step.
"""
import numpy as np
import pytest

import workloads as W
from kvc_testlib import mask_bits
from oracle import policy, regions

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

F32_MAX = float(np.finfo(np.float32).max)


@pytest.fixture(scope="module", autouse=True)
def _needs_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def kvc():
    import decode_attention_compressed_quantize_amd as m

    return m


def special_scores(kind, shape, seed):
    rng = np.random.default_rng(seed)
    if kind == "ties":  # a few values only: long runs of equal keys
        return rng.integers(-1, 3, size=shape).astype(np.float32)
    s = rng.standard_normal(shape).astype(np.float32)
    flat = s.reshape(-1)
    n = flat.size
    for value, frac in ((np.nan, 0.02), (np.inf, 0.01), (-np.inf, 0.01), (-0.0, 0.05), (0.0, 0.05)):
        flat[rng.integers(0, n, max(1, int(frac * n)))] = value
    return s


def _check_mask(c, lengths, scores, budget, what):
    words = c.keep_mask.cpu().numpy()
    nbits = words.shape[-1] * 32
    for b, L in enumerate(lengths):
        start, n4 = regions.int4_range(int(L))
        for h in range(scores.shape[1]):
            want = np.zeros(nbits, bool)
            want[regions.int8_positions(int(L))] = True
            want[start:start + n4] = policy.topk_keep(scores[b, h, start:start + n4], budget)
            got = mask_bits(words[b, h], nbits)
            bad = np.flatnonzero(got != want)
            assert bad.size == 0, f"{what} b={b} h={h} L={L}: {bad.size} bits differ, first {bad[:8]}"


@pytest.mark.parametrize("kind", ["ties", "special"])
@pytest.mark.parametrize("budget", [0, 1, 123, 300, 500, 999, 1000])
@pytest.mark.parametrize("stateful", [False, True])
def test_token_topk_given_special_scores(kind, budget, stateful):
    """Caller-written scores: every call is a full refresh (radix select over
    order keys, in-order tie pass); with a state the lists are rebuilt too."""
    m = kvc()
    lengths = [0, 1, 100, 144, 145, 146, 161, 1000, 5000, 70000]
    max_ctx = 70000
    nseq, hkv = len(lengths), 2
    scores = special_scores(kind, (nseq, hkv, max_ctx), seed=budget * 7 + (kind == "ties"))
    pages = (max_ctx + 15) // 16
    table = torch.arange(nseq * pages, dtype=torch.int32, device="cuda").view(nseq, pages)
    seq = torch.tensor(lengths, dtype=torch.int32, device="cuda")
    c = m.Cache(nseq, hkv, 64, max_ctx, nseq * pages, table, seq)
    c.keep_mask.fill_(-1)
    c.scores.copy_(torch.from_numpy(scores))
    state = m.topk_workspace(c) if stateful else None
    print(f"token top-k given scores kind={kind} budget={budget} state={stateful}", flush=True)
    for rep in range(2 if stateful else 1):
        m.kvc_score_topk_mask(c, None, None, None, None, budget, ws=state)
        torch.cuda.synchronize()
        _check_mask(c, lengths, scores, budget, f"{kind}/{budget}/rep{rep}")


def special_mlp(D):
    """Two heads of scorer weights whose float32 evaluation yields special values.

    Hidden unit u reads one input coordinate (W1 row = one-hot), so
    h_u = x_j + b1_u with x_j a unit-normal source entry.
    Head 0: +-FLT_MAX output weights overflow to +-inf, two units on the same
    coordinate with opposite huge weights cancel to NaN (inf - inf) or 0, and
    a plain unit relu(x_3) gives distinct positive scores; tokens where every
    unit is inactive score +0 (long runs of ties).
    Head 1: non-positive weights: -relu(x_0) (-0 or negative), -inf from a
    huge negative weight; b2 = -0.
    """
    H = 32
    per = H * 2 * D + 2 * H + 1
    w = np.zeros((2, per), np.float32)

    def unit(h, u, j, b1, w2):
        w[h, u * 2 * D + j] = 1.0
        w[h, H * 2 * D + u] = b1
        w[h, H * 2 * D + H + u] = w2

    unit(0, 0, 0, -1.0, F32_MAX)
    unit(0, 1, 1, -1.0, -F32_MAX)
    unit(0, 2, 2, -0.5, F32_MAX)
    unit(0, 3, 2, -0.5, -F32_MAX)
    unit(0, 4, 3, 0.0, 1.0)
    unit(0, 5, D + 5, 0.0, 0.25)  # a V coordinate too
    unit(1, 0, 0, 0.0, -1.0)
    unit(1, 1, 1, -1.5, -F32_MAX)
    unit(1, 2, D + 7, -0.2, -0.5)
    w[1, -1] = -0.0
    return w


def test_incremental_topk_on_special_mlp_scores():
    """Decode steps with the refresh state while the MLP produces +-inf, NaN,
    +-0 and ties; the budget moves once (300 -> 700 per mille). The mask must
    equal the oracle's top-k of the GPU's own scores after every step, and the
    state must have taken the incremental update on most steps."""
    m = kvc()
    from decode_attention_compressed_quantize_amd.workload_cache import LayerCache

    w = W.WORKLOADS["fullstep"].replace(name="special_mlp", batch=3, kv_heads=2, q_heads=8,
                                        layers=1, ctx=3000, ctx_list=(400, 1500, 3000),
                                        decode_steps=260)
    lc = LayerCache(w)
    D = w.head_dim
    mlp = torch.from_numpy(special_mlp(D)).cuda()
    # re-score the prefill with the special scorer (positions [0, L) of every sequence)
    lmax = int(lc.lengths.max())
    k_all = torch.zeros((w.batch, lmax, w.kv_heads, D), dtype=torch.bfloat16, device="cuda")
    v_all = torch.zeros_like(k_all)
    for b in range(w.batch):
        L = int(lc.lengths[b])
        k_all[b, :L] = lc.k_src[b]
        v_all[b, :L] = lc.v_src[b]
    n_all = torch.from_numpy(lc.lengths.astype(np.int32)).cuda()
    state = m.topk_workspace(lc.cache)
    budget_of = lambda s: 300 if s < 130 else 700
    m.kvc_score_topk_mask(lc.cache, mlp, k_all, v_all, n_all, budget_of(0), ws=state)
    del k_all, v_all
    lens = lc.lengths.copy()
    one = torch.ones(w.batch, dtype=torch.int32, device="cuda")
    kinds = {"nan": 0, "+inf": 0, "-inf": 0, "-0": 0, "+0": 0}
    incremental = 0
    prev_nanb = None
    for step in range(260):
        budget = budget_of(step)
        k_new = W.kv_rows_torch(w, 0, "K", lens, "cuda")[:, None]
        v_new = W.kv_rows_torch(w, 0, "V", lens, "cuda")[:, None]
        lens += 1
        lc.seq_lens.copy_(torch.from_numpy(lens.astype(np.int32)))
        if step % 2:
            m.kvc_append_score_topk_mask(lc.cache, mlp, k_new, v_new, one, budget, ws=state)
        else:
            m.kvc_quantize_append(lc.cache, k_new, v_new, one)
            m.kvc_score_topk_mask(lc.cache, mlp, k_new, v_new, one, budget, ws=state)
        torch.cuda.synchronize()
        scores = lc.cache.scores.cpu().numpy()
        _check_mask(lc.cache, lens, scores, budget, f"step {step}")
        st = state.cpu().numpy().reshape(w.batch * w.kv_heads, -1)
        nanb = st[:, 4:6].copy()
        if prev_nanb is not None:
            # an incremental step moves each list length by at most one; a full refresh refills them
            incremental += int((np.abs(nanb - prev_nanb).max(axis=1) <= 1).sum())
        prev_nanb = nanb
    for b in range(w.batch):
        s = scores[b, :, :int(lens[b])].reshape(-1)
        kinds["nan"] += int(np.isnan(s).sum())
        kinds["+inf"] += int(np.isposinf(s).sum())
        kinds["-inf"] += int(np.isneginf(s).sum())
        kinds["-0"] += int(((s == 0) & np.signbit(s)).sum())
        kinds["+0"] += int(((s == 0) & ~np.signbit(s)).sum())
    print(f"special scores seen: {kinds}; pair-steps consistent with the incremental update: "
          f"{incremental} of {259 * w.batch * w.kv_heads}", flush=True)
    for kname in ("nan", "+inf", "-inf", "+0"):
        assert kinds[kname] > 0, f"the scorer produced no {kname}"
    assert incremental > 259 * w.batch * w.kv_heads // 2
