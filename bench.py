#!/usr/bin/env python3
"""Benchmark: decode steps over a compressed KV cache on one MI355X.

A step is one pass of the whole hot path over one batch: append one bf16 K/V
token per sequence (INT4 + INT8 ring encode), score it with the per-head MLP
and refresh the top-k keep mask, then the split INT4/INT8 decode attention
with the log-sum-exp merge. Inputs (new tokens, queries) are generated and
resident in HBM before the timed region.

Default workload ``long128k``: batch 4, 32 query / 8 kv heads, head_dim 128,
context 131072, keep masks from a seeded per-head MLP at 10% and at 50%
(one cache per budget; a step runs both). To keep the 256 MB Infinity Cache
from serving repeated reads, steps rotate over replica caches so that more
than 1 GiB of cache is touched between two reads of the same replica.

Prints one JSON line. ``value`` is KV GB/s: the attention's algorithmic bytes
per step (kept INT4 tokens at 160 B, INT8 tokens at 264 B per kv head, plus
queries, outputs, mask words and block table) divided by the whole step time.
"""
from __future__ import annotations

import argparse
import json
import statistics
import math
import os
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
HOST_LINK_PEAK_GBS = 64.0  # PCIe Gen5 x16, one direction
# Host tier: "cold" demotes pages whose positions are all evicted after the
# prefill; "all" moves every whole INT4-region page to the host tier.
TIER_MODE = {"long128k_tiered": "cold", "long128k_streamed": "all"}
# rocprofv3 PMC summaries of the attention call: workload -> (summary, kernel source it was taken with)
_CSRC = os.path.join(ROOT, "decode_attention_compressed_quantize_amd", "csrc")
TRAFFIC = {
    "long128k": (os.path.join(ROOT, "profiles", "attention_long128k_traffic.txt"),
                 os.path.join(_CSRC, "attention.hip")),
    "long128k_dense": (os.path.join(ROOT, "profiles", "attention_long128k_dense_traffic.txt"),
                       os.path.join(_CSRC, "dense_attention.hip")),
}

WORKLOAD_LAYERS = {
    "long128k": ["long128k_b10", "long128k_b50"],
    "long128k_blocks": ["long128k_blk_b10", "long128k_blk_b50"],
    "long128k_recent16k": ["long128k_r16k_b10", "long128k_r16k_b50"],
    "long128k_kv4": ["long128k_kv4_b10", "long128k_kv4_b50"],
    "long128k_tiered": ["long128k_blk_b10", "long128k_blk_b50"],
    "long128k_streamed": ["long128k_b10"],
    "uniform4k": ["uniform4k"],
    "longtail": ["longtail"],
    "fullstep": ["fullstep"] * 36,
    "tiny": ["tiny"],
}
# The uncompressed baseline: a dense bfloat16 paged cache of the same shape as
# long128k (two layers per step), every position attended.
DENSE = {"long128k_dense": dict(batch=4, q_heads=32, kv_heads=8, head_dim=128, ctx=131072, layers=2)}


def algorithmic_bytes(w, lengths, keep4_counts):
    """Bytes one attention call must move for workload ``w`` at ``lengths``."""
    D, Hkv, Hq = w.head_dim, w.kv_heads, w.q_heads
    per4 = D + 8 * (D // 32)          # K+V codes + K/V scale,min per group
    per8 = 2 * D + 8                  # K+V int8 codes + two fp32 scales
    qbytes = 2 if w.src_dtype == "bf16" else 4
    total = 0
    sink, recent = (16, 128) if w.protect else (0, 0)
    for b, L in enumerate(lengths):
        L = int(L)
        n8 = min(L, sink) + max(0, L - max(sink, L - recent)) if w.protect else 0
        n4 = max(0, L - sink - recent)
        total += Hkv * n8 * per8 + int(keep4_counts[b]) * per4
        if w.recency_window > 0:  # the windowed call reads only the window's words and pages
            nw = min(n4, w.recency_window)
            total += Hkv * ((nw + 31) // 32) * 4
            total += ((nw + 15) // 16) * 4
        else:
            total += Hkv * ((sink + n4 + 31) // 32) * 4   # mask words over the INT4 region
            total += ((L + 15) // 16) * 4                 # block table entries
        total += Hq * (D * qbytes + D * 4 + 4)        # q in, out and lse
    return total


def kept_counts(w, lengths):
    """Kept INT4 positions summed over kv heads, per sequence.

    Under the block policy only the first and the last candidate block can
    hold fewer than ``block_tokens`` positions (at least one each), so the
    count used is the lower bound (kb - 2) * B + 2, never an overstatement."""
    out = []
    slots = 144 if w.protect else 0
    for L in lengths:
        n4 = max(0, int(L) - slots)
        if w.mask == "all":
            k = n4
        elif w.mask in ("scores", "mlp") and w.policy == "block":
            B = w.block_tokens
            c0 = max(0, n4 - w.recency_window) if w.recency_window > 0 else 0
            nb = (n4 + B - 1) // B - c0 // B if n4 > c0 else 0
            kb = (w.budget_permille * nb) // 1000
            k = n4 - c0 if kb >= nb else max(kb, kb * B - 2 * (B - 1))
        elif w.mask in ("scores", "mlp"):
            k = (w.budget_permille * n4) // 1000
        else:
            k = n4 // 2
        out.append(k * w.kv_heads)
    return out


def measured_traffic(workload: str):
    """HBM bytes per attention call from the committed rocprofv3 PMC summary.

    The summary records FETCH_SIZE and WRITE_SIZE per dispatch of the two
    attention launches, already scaled by the copy-kernel calibration, and
    the sha256 of the kernel source they were taken with; returns None when
    the source has changed since or the workload differs.
    """
    import hashlib

    if workload not in TRAFFIC or not os.path.exists(TRAFFIC[workload][0]):
        return None
    summary, source = TRAFFIC[workload]
    fields = {}
    with open(summary) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                fields[k.strip()] = v.strip()
    src = hashlib.sha256(open(source, "rb").read()).hexdigest()
    if fields.get("kernel_source_sha256") != src:
        return None
    try:
        return float(fields["hbm_bytes_per_call"])
    except (KeyError, ValueError):
        return None


def read_ceiling_gbs():
    """The streaming-read rate of this GPU: kvc_stream_read_probe over a 4 GiB buffer
    (16-byte loads, every word read once), median of 10 calls between HIP events."""
    import torch

    import decode_attention_compressed_quantize_amd as kvc

    buf = torch.empty(1 << 30, dtype=torch.int32, device="cuda")
    out = torch.zeros(1, dtype=torch.int32, device="cuda")
    for _ in range(3):
        kvc.kvc_stream_read_probe(buf, out)
    ts = []
    for _ in range(10):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        kvc.kvc_stream_read_probe(buf, out)
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    del buf
    return (4 << 30) / (statistics.median(ts) * 1e-3) / 1e9


def add_read_ceiling(line, ceil=None):
    """Also state the attention call's rate against the measured streaming-read ceiling."""
    if ceil is None:
        ceil = read_ceiling_gbs()
    line["roofline"]["read_ceiling_GBs"] = round(ceil, 1)
    line["roofline"]["frac_of_read_ceiling"] = round(line["roofline"]["achieved"] / ceil, 4)


# ---------------------------------------------------------------------- CPU
def _cpu_pair(args):
    """Oracle attention phase for one (workload, b, kvh): returns (bytes, seconds)."""
    name, b, kvh = args
    from threadpoolctl import threadpool_limits

    import numpy as np

    import workloads as W
    from oracle import attention, policy, reference, regions

    with threadpool_limits(1):
        w = W.WORKLOADS[name]
        L = int(w.lengths()[b])
        k = W.bf16_bits_to_f32(W.kv_source_np(w, 0, "K", b, 0, L, kvh=kvh))
        v = W.bf16_bits_to_f32(W.kv_source_np(w, 0, "V", b, 0, L, kvh=kvh))
        ns, nr = (regions.N_SINK, regions.N_RECENT) if w.protect else (0, 0)
        enc = reference.encode(k, v, ns, nr)
        start, n4 = regions.int4_range(L, ns, nr)
        if w.mask == "mlp":
            s = policy.mlp_scores(k, v, W.mlp_weights(w, 0)[kvh])
            if w.policy == "block":
                keep4 = policy.block_keep(s[start:start + n4], w.budget_permille, w.block_tokens,
                                          w.recency_window)
            else:
                keep4 = policy.topk_keep(s[start:start + n4], w.budget_permille)
        else:
            keep4 = np.ones(n4, bool)
        G = w.group_size
        q = W.bf16_bits_to_f32(W.queries_np(w, 0, 0)[b, kvh * G:(kvh + 1) * G]).astype(np.float64)
        t0 = time.perf_counter()
        kh, vh = reference.decoded(enc)
        pos = reference.kept_positions(L, keep4, ns, nr)
        attention.attend(q, kh[pos], vh[pos])
        dt = time.perf_counter() - t0
        n8 = len(regions.int8_positions(L, ns, nr))
        nbytes = int(keep4.sum()) * (w.head_dim + 8 * (w.head_dim // 32)) + n8 * (2 * w.head_dim + 8)
        return nbytes, dt


def cpu_baseline(layer_names, seconds: float):
    """Time the oracle's attention phase over a bounded sample of (sequence, kv head) pairs."""
    import multiprocessing as mp

    import workloads as W

    cores = len(os.sched_getaffinity(0))
    cores = max(1, min(cores, 16))
    pairs = []
    i = 0
    for name in layer_names[:2]:
        w = W.WORKLOADS[name]
        for b in range(w.batch):
            for h in range(w.kv_heads):
                pairs.append((name, b, h))
    # bounded sample: interleave layers, take enough pairs for ~`seconds` of work
    probe = _cpu_pair(pairs[0])
    per_pair = max(probe[1], 1e-3)
    n = int(min(len(pairs), max(cores, seconds * cores / per_pair)))
    step = max(1, len(pairs) // n)
    sample = pairs[::step][:n]
    ctx = mp.get_context("spawn")
    with ctx.Pool(min(cores, len(sample))) as pool:
        res = pool.map(_cpu_pair, sample)
    used = min(cores, len(sample))
    nbytes = sum(r[0] for r in res)
    busy = sum(r[1] for r in res)
    gbs = nbytes / (busy / used) / 1e9
    return {"value": round(gbs, 4), "unit": "GB/s", "cores": used, "kind": "oracle",
            "sample": f"{len(sample)} (sequence, kv head) pairs of {'+'.join(sorted(set(layer_names[:2])))}: "
                      f"float64 decode + masked softmax attention, busy time summed over "
                      f"{used} worker processes (1 thread each) and divided by {used}"}


# ---------------------------------------------------------------------- dense baseline
def dense_bytes(w, lengths):
    """Bytes one dense attention call must move: every position's K and V rows in
    bfloat16, the block table, queries, outputs and LSE."""
    D, Hkv, Hq = w.head_dim, w.kv_heads, w.q_heads
    total = 0
    for L in lengths:
        L = int(L)
        total += Hkv * L * 4 * D + ((L + 15) // 16) * 4 + Hq * (D * 2 + D * 4 + 4)
    return total


def _cpu_dense_pair(args):
    """Oracle dense attention for one (workload, b, kvh): returns (bytes, seconds)."""
    name, b, kvh = args
    from threadpoolctl import threadpool_limits

    import numpy as np

    import workloads as W
    from oracle import dense

    with threadpool_limits(1):
        cfg = DENSE[name]
        w = W.Workload(name, cfg["batch"], cfg["q_heads"], cfg["kv_heads"], cfg["head_dim"],
                       ctx=cfg["ctx"])
        L = int(w.lengths()[b])
        k = W.bf16_bits_to_f32(W.kv_source_np(w, 0, "K", b, 0, L, kvh=kvh))
        v = W.bf16_bits_to_f32(W.kv_source_np(w, 0, "V", b, 0, L, kvh=kvh))
        G = w.group_size
        q = W.bf16_bits_to_f32(W.queries_np(w, 0, 0)[b, kvh * G:(kvh + 1) * G]).astype(np.float64)
        t0 = time.perf_counter()
        dense.decode_group(q, k, v, "bf16")
        return L * 4 * w.head_dim, time.perf_counter() - t0


def dense_main(args):
    import numpy as np
    import torch

    import workloads as W
    import decode_attention_compressed_quantize_amd as kvc
    from decode_attention_compressed_quantize_amd.workload_cache import DenseLayerCache

    kvc.lib()
    cfg = DENSE[args.workload]
    total_steps = args.warmup + args.steps
    print(f"bench: building {args.workload} ({cfg['layers']} dense layer caches)", file=sys.stderr,
          flush=True)
    layers = []
    for li in range(cfg["layers"]):
        w = W.Workload(args.workload, cfg["batch"], cfg["q_heads"], cfg["kv_heads"], cfg["head_dim"],
                       ctx=cfg["ctx"], decode_steps=total_steps + 1)
        layers.append(DenseLayerCache(w, layer=li))
    for lc in layers[1:]:  # the layers of one batch share one lengths tensor
        lc.seq_lens = layers[0].seq_lens
        lc.cache.seq_lens = layers[0].seq_lens
        lc.cache.desc.seq_lens = layers[0].seq_lens.data_ptr()
    dev = "cuda"
    inputs = []
    for li, lc in enumerate(layers):
        w = lc.w
        L0 = lc.lengths.copy()
        ks, vs, qs = [], [], []
        for s in range(total_steps + 1):
            ks.append(W.kv_rows_torch(w, li, "K", L0 + s, dev)[:, None])
            vs.append(W.kv_rows_torch(w, li, "V", L0 + s, dev)[:, None])
            qs.append(W.queries_torch(w, li, s + 1, dev))
        inputs.append({"k": ks, "v": vs, "q": qs, "ws": lc.workspace(),
                       "out": torch.empty((w.batch, w.q_heads, w.head_dim), dtype=torch.float32, device=dev),
                       "lse": torch.empty((w.batch, w.q_heads), dtype=torch.float32, device=dev),
                       "one": torch.ones(w.batch, dtype=torch.int32, device=dev)})
    lens = layers[0].lengths.astype(np.int64).copy()
    stream = torch.cuda.current_stream()
    TIME_EVERY = 4
    attn = []

    def step(i, record):
        layers[0].seq_lens.add_(1)
        lens[:] += 1
        byts = 0
        for li, lc in enumerate(layers):
            st = inputs[li]
            lc.append(st["k"][i], st["v"][i], st["one"])
            if record:
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
            kvc.kvc_dense_decode_attention(lc.cache, st["q"][i], st["out"], st["lse"], st["ws"])
            if record:
                e1.record(stream)
                attn.append((e0, e1))
            byts += dense_bytes(lc.w, lens)
        return byts

    for i in range(args.warmup):
        step(i, False)
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    step_bytes = 0
    t0.record(stream)
    for i in range(args.warmup, total_steps):
        step_bytes += step(i, (i - args.warmup) % TIME_EVERY == 0)
    t1.record(stream)
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / args.steps
    gbs = step_bytes / args.steps / (ms * 1e-3) / 1e9
    a_ms = statistics.median(e0.elapsed_time(e1) for e0, e1 in attn)
    a_bytes = dense_bytes(layers[0].w, lens)
    a_gbs = a_bytes / (a_ms * 1e-3) / 1e9
    print(f"bench: dense attention call times (ms): " +
          " ".join(f"{e0.elapsed_time(e1):.4f}" for e0, e1 in attn), file=sys.stderr, flush=True)
    w = layers[0].w
    line = {
        "metric": "dense bf16 KV decode attention (uncompressed baseline): KV bytes GB/s (% HBM peak), decode steps/s",
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 K/V, bf16 MFMA logits (two-part query), f32 P.V and accumulate",
        "data": "synthetic (seeded normal K/V/Q)",
        "config": {"workload": args.workload, "layers": f"{cfg['layers']} x dense bf16",
                   "batch": w.batch, "q_heads": w.q_heads, "kv_heads": w.kv_heads,
                   "head_dim": w.head_dim, "context": cfg["ctx"], "replicas": 1,
                   "keep_policy": "none (every position attended)"},
        "decode_steps_per_s": round(1000.0 / ms, 2),
        "pct_hbm_peak": round(100.0 * gbs / HBM_PEAK_GBS, 2),
        "attention": {"ms_per_call": round(a_ms, 5), "GBs": round(a_gbs, 1), "timed_calls": len(attn),
                      "timed_every_nth_step": TIME_EVERY, "statistic": "median call time"},
        "roofline": {"kernel": "kvc_dense_decode_attention call: dense_attention_kernel then "
                               "merge_kernel, timed together with HIP events on the launch stream",
                     "bound": "hbm", "achieved": round(a_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(a_gbs / HBM_PEAK_GBS, 4), "traffic": measured_traffic(args.workload),
                     "algorithmic_bytes_per_call": int(a_bytes)},
        "cpu_baseline": None,
    }
    add_read_ceiling(line)
    if not args.no_cpu:
        import multiprocessing as mp

        print("bench: timing the CPU oracle sample", file=sys.stderr, flush=True)
        cores = max(1, min(len(os.sched_getaffinity(0)), 16))
        sample = [(args.workload, b, h) for b in range(w.batch) for h in range(w.kv_heads)][:cores]
        with mp.get_context("spawn").Pool(len(sample)) as pool:
            res = pool.map(_cpu_dense_pair, sample)
        busy = sum(r[1] for r in res)
        line["cpu_baseline"] = {
            "value": round(sum(r[0] for r in res) / (busy / len(sample)) / 1e9, 4), "unit": "GB/s",
            "cores": len(sample), "kind": "oracle",
            "sample": f"{len(sample)} (sequence, kv head) pairs of {args.workload}: float64 dense "
                      f"softmax attention over bf16 rows, busy time summed over {len(sample)} "
                      f"worker processes (1 thread each) and divided by {len(sample)}"}
    print(json.dumps(line), flush=True)


# ---------------------------------------------------------------------- learner
# Learner-side shadow-mask attention: B sequences of a prompt plus generated
# positions whose keep masks come from a rollout recorded on the GPU (one
# layer, per-head MLP scores, top-30% refresh every step). A step is one
# kvc_shadow_attention call over the batch.
LEARNER = {"learner8k": dict(batch=4, prompt=4096, generated=4096, q_heads=32, kv_heads=8,
                             head_dim=128, budget_permille=300)}


def _learner_pairs(rows_np, prompts, lens, kv_heads):
    """Attended (kv head, query position, key) triples: dense causal prompt rows plus
    each generated row's kept positions up to itself."""
    import numpy as np

    total = 0
    for b in range(len(lens)):
        P, L = int(prompts[b]), int(lens[b])
        total += kv_heads * P * (P + 1) // 2
        bits = np.unpackbits(np.ascontiguousarray(rows_np[b]).view(np.uint8), axis=-1,
                             bitorder="little")
        for r in range(L - P):
            total += int(bits[:, r, : P + r + 1].sum())
    return total


def _learner_cpu(cfg, w, q, k, v, prompts, rows_np, seconds):
    """Oracle rows on a bounded sample: float64 masked softmax attention per row."""
    import numpy as np

    from oracle import shadow as oshadow
    from oracle import attention

    G = cfg["q_heads"] // cfg["kv_heads"]
    qn = q[0].float().cpu().numpy().astype(np.float64)
    kn = k[0].float().cpu().numpy().astype(np.float64)
    vn = v[0].float().cpu().numpy().astype(np.float64)
    P = int(prompts[0])
    bits = np.unpackbits(np.ascontiguousarray(rows_np[0]).view(np.uint8), axis=-1, bitorder="little")
    rng = np.random.default_rng(0)
    flops = 0
    n = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        p = int(rng.integers(P, qn.shape[0]))
        for g in range(cfg["kv_heads"]):
            pos = oshadow.allowed_positions(p, P, bits[g, p - P].astype(bool))
            hs = slice(g * G, (g + 1) * G)
            attention.attend(qn[p, hs], kn[pos, g], vn[pos, g])
            flops += G * len(pos) * 4 * cfg["head_dim"]
        n += 1
    dt = time.perf_counter() - t0
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": 1, "kind": "oracle",
            "sample": f"{n} generated query positions of sequence 0 (all {cfg['q_heads']} heads), "
                      f"float64 masked softmax attention, one thread"}


def learner_main(args):
    import numpy as np
    import torch

    import workloads as W
    import decode_attention_compressed_quantize_amd as kvc
    from decode_attention_compressed_quantize_amd.workload_cache import LayerCache

    kvc.lib()
    cfg = LEARNER[args.workload]
    w = W.Workload(args.workload, cfg["batch"], cfg["q_heads"], cfg["kv_heads"], cfg["head_dim"],
                   ctx=cfg["prompt"], mask="mlp", budget_permille=cfg["budget_permille"],
                   decode_steps=cfg["generated"])
    print(f"bench: recording a {cfg['generated']}-step rollout", file=sys.stderr, flush=True)
    lc = LayerCache(w, keep_sources=False)
    prompts = lc.lengths.copy()
    rows, lens = lc.record_rollout(cfg["generated"], ws=lc.refresh_state())
    T = int(lens.max())
    B, Hq, Hkv, D = cfg["batch"], cfg["q_heads"], cfg["kv_heads"], cfg["head_dim"]
    q = torch.empty((B, T, Hq, D), dtype=torch.bfloat16, device="cuda")
    k = torch.empty((B, T, Hkv, D), dtype=torch.bfloat16, device="cuda")
    v = torch.empty_like(k)
    for b in range(B):
        q[b] = W.learner_queries_torch(w, 0, b, 0, T, "cuda")
        k[b] = W.kv_source_torch(w, 0, "K", b, 0, T, "cuda")
        v[b] = W.kv_source_torch(w, 0, "V", b, 0, T, "cuda")
    out = torch.empty((B, T, Hq, D), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, T, Hq), dtype=torch.float32, device="cuda")
    sl = torch.tensor(lens.astype(np.int32), device="cuda")
    pl = torch.tensor(prompts.astype(np.int32), device="cuda")
    rows_np = rows.cpu().numpy()
    pairs = _learner_pairs(rows_np, prompts, lens, Hkv)
    flops = pairs * (Hq // Hkv) * 4 * D  # QK^T and PV: 2D + 2D per attended (query head, key)
    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        kvc.kvc_shadow_attention(q, k, v, sl, pl, rows, out, lse)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        kvc.kvc_shadow_attention(q, k, v, sl, pl, rows, out, lse)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    tflops = flops / (ms * 1e-3) / 1e12
    kept = pairs / (Hkv * sum(int(L) * (int(L) + 1) // 2 for L in lens))
    line = {
        "metric": "learner shadow-mask attention: useful TFLOP/s (attended pairs x 4D)",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 MFMA operands, f32 accumulate",
        "data": "synthetic (seeded normal Q/K/V; shadow rows recorded from a GPU rollout with seeded MLP scores)",
        "config": {"workload": args.workload, "batch": B, "prompt": cfg["prompt"],
                   "generated": cfg["generated"], "q_heads": Hq, "kv_heads": Hkv, "head_dim": D,
                   "keep_policy": f"token, budget {cfg['budget_permille'] / 10:g}% (generated rows)",
                   "attended_fraction_of_causal": round(kept, 4)},
        "roofline": {"kernel": "shadow_attention_kernel (one launch)", "bound": "mfma",
                     "achieved": round(tflops, 1), "peak": 2500.0, "unit": "TFLOP/s",
                     "frac": round(tflops / 2500.0, 4), "traffic": None,
                     "useful_flops_per_call": int(flops)},
        "cpu_baseline": None,
    }
    if not args.no_cpu:
        print("bench: timing the CPU oracle sample", file=sys.stderr, flush=True)
        line["cpu_baseline"] = _learner_cpu(cfg, w, q, k, v, prompts, rows_np, args.cpu_seconds)
    print(json.dumps(line), flush=True)


# ---------------------------------------------------------------------- GPU
def decode_run(args, workload, steps, warmup, calls, reps, pool_mode="auto", replicas_arg=0):
    """Build one workload's caches (with replicas), run ``warmup`` + ``steps`` timed decode
    steps, then time the attention call alone: ``reps`` repetitions of ``calls`` calls per
    layer, rotating over the replicas as the steps do. Returns the measurements."""
    import numpy as np
    import torch

    import workloads as W
    import decode_attention_compressed_quantize_amd as kvc
    from decode_attention_compressed_quantize_amd.workload_cache import LayerCache

    kvc.lib()
    dev = "cuda"
    names = WORKLOAD_LAYERS[workload]
    total_steps = warmup + steps
    base = [W.WORKLOADS[n].replace(decode_steps=total_steps + 1) for n in names]
    per_replica_bytes = 0
    layers = []
    print(f"bench: building {workload} ({len(base)} layer caches per replica)", file=sys.stderr, flush=True)
    tier = TIER_MODE.get(workload)
    host_moved = 0

    def pooled(w):
        # auto: the token policy; the block policy maintains a pool too (--pool on),
        # but at 128K its refresh launch then costs more than the attention saves
        if pool_mode == "off" or tier:
            return False
        if w.recency_window != 0 or w.mask not in ("mlp", "scores", "all"):
            return False
        return w.policy == "token" or (w.policy == "block" and pool_mode == "on")

    for li, w in enumerate(base):
        host = W.page_table(w, li)[1] if tier else 0
        lc = LayerCache(w, layer=li, device=dev, keep_sources=False, host_pages=host,
                        pool=pooled(w))
        if tier == "cold":
            host_moved += lc.demote_cold_pages()
        elif tier == "all":
            host_moved += lc.stream_int4_region()
        layers.append(lc)
        per_replica_bytes += lc.cache.nbytes()
    replicas = replicas_arg
    read_per_replica = sum(algorithmic_bytes(lc.w, lc.lengths, kept_counts(lc.w, lc.lengths))
                           for lc in layers)
    if replicas <= 0:
        replicas = max(1, math.ceil((1 << 30) / read_per_replica) + 1) if len(base) < 8 else 1
    if tier == "all":
        replicas = 1  # host-tier reads are not served by the GPU's caches
    # replicas are device copies of the prefilled caches, within 96 GiB in all
    replicas = max(1, min(replicas, int((96 << 30) // max(1, per_replica_bytes))))
    reps_c = [layers]
    for r in range(1, replicas):
        reps_c.append([lc.replica() for lc in layers])
    # As in a model, the layers of one batch share one lengths tensor, which the
    # caller advances once per step.
    for rep in reps_c:
        for lc in rep[1:]:
            assert np.array_equal(lc.lengths, rep[0].lengths)
            lc.seq_lens = rep[0].seq_lens
            lc.cache.seq_lens = rep[0].seq_lens
            lc.cache.desc.seq_lens = rep[0].seq_lens.data_ptr()
    print(f"bench: {replicas} replica(s), {per_replica_bytes / 2**30:.2f} GiB each", file=sys.stderr, flush=True)

    # inputs for every step, resident before timing
    inputs = []
    for r, rep in enumerate(reps_c):
        per = []
        for li, lc in enumerate(rep):
            w = lc.w
            steps_here = (total_steps + replicas - 1) // replicas + 1
            L0 = lc.lengths.copy()
            ks, vs, qs = [], [], []
            for s in range(steps_here):
                ks.append(W.kv_rows_torch(w, li, "K", L0 + s, dev)[:, None])
                vs.append(W.kv_rows_torch(w, li, "V", L0 + s, dev)[:, None])
                qs.append(W.queries_torch(w, li, s + 1, dev))
            out = torch.empty((w.batch, w.q_heads, w.head_dim), dtype=torch.float32, device=dev)
            lse = torch.empty((w.batch, w.q_heads), dtype=torch.float32, device=dev)
            per.append({"k": ks, "v": vs, "q": qs, "out": out, "lse": lse, "ws": lc.workspace(),
                        "state": lc.refresh_state(),
                        "one": torch.ones(w.batch, dtype=torch.int32, device=dev),
                        "lens": lc.lengths.astype(np.int64).copy(), "n": 0})
        inputs.append(per)

    stream = torch.cuda.current_stream()

    def attend(lc, st, s):
        w = lc.w
        if w.recency_window > 0:
            kvc.kvc_decode_attention_windowed(lc.cache, w.recency_window, st["q"][s], st["out"],
                                              st["lse"], st["ws"])
        else:
            kvc.kvc_decode_attention(lc.cache, st["q"][s], st["out"], st["lse"], st["ws"])

    def step(i):
        r = i % replicas
        byts = 0
        reps_c[r][0].seq_lens.add_(1)
        for li, lc in enumerate(reps_c[r]):
            st = inputs[r][li]
            s = st["n"]
            st["n"] += 1
            st["lens"] += 1
            lc.append_refresh(st["k"][s], st["v"][s], st["one"], ws=st["state"])
            attend(lc, st, s)
            byts += algorithmic_bytes(lc.w, st["lens"], kept_counts(lc.w, st["lens"]))
        return byts

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    step_bytes = 0
    t0.record(stream)
    for i in range(warmup, warmup + steps):
        step_bytes += step(i)
    t1.record(stream)
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps
    gbs = step_bytes / steps / (ms * 1e-3) / 1e9

    # the attention call alone: each call between two HIP events on the launch
    # stream, `calls` calls per layer and repetition, replicas in rotation (the
    # layers interleaved as in a step), caches as the last step left them
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(calls)] for _ in names]
    per_layer_t = {}  # layer name -> per repetition, the call times (layers of one name pooled)
    for rep in range(reps):
        for j in range(calls):
            r = (rep * calls + j) % replicas
            for li, lc in enumerate(reps_c[r]):
                st = inputs[r][li]
                e0, e1 = ev[li][j]
                e0.record(stream)
                attend(lc, st, max(0, st["n"] - 1))
                e1.record(stream)
        torch.cuda.synchronize()
        times = {}
        for li, lc in enumerate(reps_c[0]):
            times.setdefault(lc.w.name, []).extend(e0.elapsed_time(e1) for e0, e1 in ev[li])
        for n, t in times.items():
            per_layer_t.setdefault(n, []).append(t)
    call_bytes = {}
    for li, lc in enumerate(reps_c[0]):
        call_bytes[lc.w.name] = algorithmic_bytes(lc.w, inputs[0][li]["lens"],
                                                  kept_counts(lc.w, inputs[0][li]["lens"]))
    per_layer = {}
    for n, runs in per_layer_t.items():
        means = [statistics.fmean(x) for x in runs]
        flat = sorted(t for x in runs for t in x)
        med = statistics.median(means)
        peak = HOST_LINK_PEAK_GBS if tier == "all" else HBM_PEAK_GBS
        gb = call_bytes[n] / (med * 1e-3) / 1e9
        per_layer[n] = {
            "attention_ms": round(med, 5), "attention_GBs": round(gb, 1), "frac": round(gb / peak, 4),
            "rep_mean_ms_min": round(min(means), 5), "rep_mean_ms_max": round(max(means), 5),
            "call_ms_p10": round(flat[len(flat) // 10], 5), "call_ms_p90": round(flat[(9 * len(flat)) // 10], 5),
            "algorithmic_bytes": int(call_bytes[n]),
        }
    a_ms = statistics.fmean(v["attention_ms"] for v in per_layer.values())
    a_bytes = statistics.fmean(v["algorithmic_bytes"] for v in per_layer.values())
    res = {
        "names": names, "base": base, "tier": tier, "host_moved": host_moved, "layers": layers,
        "replicas": replicas, "pooled": bool(pooled(base[0])), "ms_per_step": ms, "gbs": gbs,
        "per_layer": per_layer, "a_ms": a_ms, "a_bytes": a_bytes,
        "a_gbs": a_bytes / (a_ms * 1e-3) / 1e9,
    }
    del reps_c, inputs, layers
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--workload", default="long128k",
                    choices=sorted(WORKLOAD_LAYERS) + sorted(LEARNER) + sorted(DENSE))
    ap.add_argument("--replicas", type=int, default=0, help="0 = enough for >1 GiB between reuses")
    ap.add_argument("--calls", type=int, default=50, help="attention calls per layer and repetition")
    ap.add_argument("--reps", type=int, default=7, help="repetitions of the attention-call timing")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-ceiling", action="store_true",
                    help="skip the streaming-read ceiling (a child measuring another workload)")
    ap.add_argument("--no-others", action="store_true",
                    help="skip the uniform4k / longtail figures that the default run adds")
    ap.add_argument("--pool", choices=["auto", "on", "off"], default="auto",
                    help="kept-record pool (auto: on for the token top-k policy; on: also for the "
                         "block policy; the host tier and recency windows read through the mask)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path "
              "(the kernel is measured on one GPU's share; see the sharding notes).",
              file=sys.stderr)
        sys.exit(2)
    if args.workload in LEARNER:
        learner_main(args)
        return
    if args.workload in DENSE:
        dense_main(args)
        return

    import torch

    # the streaming-read ceiling, measured before the caches take the memory
    ceil = read_ceiling_gbs() if TIER_MODE.get(args.workload) != "all" and not args.no_ceiling else None
    torch.cuda.empty_cache()
    res = decode_run(args, args.workload, args.steps, args.warmup, args.calls, args.reps, args.pool,
                     args.replicas)
    names, base, tier = res["names"], res["base"], res["tier"]
    ms, gbs = res["ms_per_step"], res["gbs"]
    a_ms, a_bytes, a_gbs = res["a_ms"], res["a_bytes"], res["a_gbs"]
    peak = HOST_LINK_PEAK_GBS if tier == "all" else HBM_PEAK_GBS
    print("bench: attention per layer: " + json.dumps(res["per_layer"]), file=sys.stderr, flush=True)
    line = {
        "metric": "compressed-KV decode attention: KV bytes GB/s (% HBM peak), decode steps/s",
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int4/int8 codes, f16 MFMA operands, f32 accumulate",
        "data": "synthetic (seeded normal K/V/Q, seeded per-head MLP scores)",
        "config": {
            "workload": args.workload,
            "layers": names if len(set(names)) > 1 else f"{len(names)} x {names[0]}",
            "batch": base[0].batch, "q_heads": base[0].q_heads, "kv_heads": base[0].kv_heads,
            "head_dim": base[0].head_dim, "context": int(base[0].lengths().max()),
            "replicas": res["replicas"],
            "kept_record_pool": res["pooled"],
            "keep_policy": [(f"{w.policy}" + (f"{w.block_tokens}" if w.policy == "block" else "")
                             + (f", recency window {w.recency_window}" if w.recency_window else "")
                             + (f", budget {w.budget_permille / 10:g}%" if w.budget_permille else ""))
                            for w in base[:2]],
        },
        "host_tier": None if not tier else {
            "mode": {"cold": "pages with every position evicted demoted after the prefill",
                     "all": "every whole INT4-region page in the host tier"}[tier],
            "pages_in_host_tier_per_replica": res["host_moved"],
            "int4_pages_per_replica": int(sum(lc.num_pages for lc in res["layers"])),
        },
        "decode_steps_per_s": round(1000.0 / ms, 2),
        "pct_hbm_peak": round(100.0 * gbs / HBM_PEAK_GBS, 2),
        "attention": {"ms_per_call": round(a_ms, 5), "GBs": round(a_gbs, 1), "per_layer": res["per_layer"],
                      "timed_calls_per_layer": args.calls * args.reps,
                      "statistic": f"per layer: median over {args.reps} repetitions of the mean of "
                                   f"{args.calls} event-timed calls (replicas in rotation); the call "
                                   f"figure averages the layers"},
        "roofline": {
            "kernel": ("kvc_decode_attention call: one attention_kernel launch (INT4 chunks over the "
                       "kept-record pool and the INT8 region, merged in-kernel), timed with HIP events "
                       "on the launch stream" if res["pooled"] else
                       "kvc_decode_attention call: attention_kernel (INT4 chunks + INT8 region) "
                       "then merge_kernel, timed together with HIP events on the launch stream"),
            "bound": "host-link" if tier == "all" else "hbm",
            "achieved": round(a_gbs, 1),
            "peak": peak,
            "unit": "GB/s",
            "frac": round(a_gbs / peak, 4),
            "traffic": measured_traffic(args.workload),
            "algorithmic_bytes_per_call": int(a_bytes),
        },
        "cpu_baseline": None,
    }
    del res
    torch.cuda.empty_cache()
    if args.workload == "long128k" and not args.no_others:
        # The other two single-GPU workloads: attention per call and the decode
        # step, each measured in a child process of its own (a fresh address
        # space, as when the workload runs alone: measured in this process after
        # the 128K caches were freed, the uniform call read ~6% slower). This
        # process holds no caches meanwhile and does no GPU work.
        others = {}
        for wl in ("uniform4k", "longtail"):
            cmd = [sys.executable, "-u", os.path.abspath(__file__), "--workload", wl, "--steps", "100",
                   "--warmup", "5", "--calls", str(args.calls), "--reps", "3", "--no-cpu", "--no-ceiling"]
            print(f"bench: measuring {wl} in a child process", file=sys.stderr, flush=True)
            r = subprocess.run(cmd, stdout=subprocess.PIPE, text=True)
            if r.returncode != 0:
                raise SystemExit(f"bench: {wl} child failed with status {r.returncode}")
            o = json.loads([ln for ln in r.stdout.splitlines() if ln.startswith("{")][-1])
            pl = next(iter(o["attention"]["per_layer"].values()))
            others[wl] = {
                "attention_us": round(1000 * pl["attention_ms"], 2), "attention_GBs": pl["attention_GBs"],
                "frac": pl["frac"], "rep_mean_us_range": [round(1000 * pl["rep_mean_ms_min"], 2),
                                                          round(1000 * pl["rep_mean_ms_max"], 2)],
                "algorithmic_bytes_per_call": pl["algorithmic_bytes"],
                "ms_per_step": o["ms_per_step"], "step_GBs": o["value"],
                "kept_record_pool": o["config"]["kept_record_pool"], "batch": o["config"]["batch"],
                "context": o["config"]["context"], "replicas": o["config"]["replicas"],
                "timing": f"100 decode steps; attention: median over 3 repetitions of {args.calls} calls; "
                          f"own process",
            }
        line["other_workloads"] = others
    if tier != "all" and not args.no_ceiling:
        add_read_ceiling(line, ceil)
    if not args.no_cpu:
        print("bench: timing the CPU oracle sample", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(names, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
