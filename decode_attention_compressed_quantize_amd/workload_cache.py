"""Build one layer's compressed cache for a synthetic workload on the GPU.

Plumbing for tests and the benchmark: inputs come from the seeded generators
in ``workloads``; all encoding, scoring, masking and attention run in libkvc
through the binding. Nothing here computes any part of the method.
"""
from __future__ import annotations

import math
from typing import Optional

import numpy as np

import workloads as W

from . import (Cache, DenseCache, attention_workspace, block_workspace, dense_workspace,
               kvc_copy_pages, kvc_dense_append, kvc_find_pages, kvc_append_score_block_mask,
               kvc_append_score_topk_mask, kvc_pool_build, kvc_quantize_append,
               kvc_score_block_mask, kvc_score_topk_mask, topk_workspace)


def pool_capacity_for(w: W.Workload) -> int:
    """Pool records per (sequence, kv head) that the workload's keep policy can need:
    its budget of the INT4 region of a max_ctx-long sequence, rounded up to 64."""
    slots = 144 if w.protect else 0
    n4max = max(0, w.max_ctx() - slots)
    if w.mask in ("scores", "mlp") and w.policy == "token":
        keep = (w.budget_permille * n4max) // 1000
    elif w.mask in ("scores", "mlp") and w.policy == "block":
        # whole blocks; with a recency window the first candidate block can be partial
        B = w.block_tokens
        span = min(w.recency_window, n4max) if w.recency_window > 0 else n4max
        nb = -(-span // B) + (1 if w.recency_window > 0 else 0)
        keep = min(n4max, (w.budget_permille * nb) // 1000 * B)
    else:
        keep = n4max
    return max(64, (keep + 63) // 64 * 64)


def pack_bits(flags: np.ndarray, words: int) -> np.ndarray:
    """Pack bool flags [n] into uint32 words (bit t%32 of word t/32) as int32."""
    out = np.zeros(words * 32, dtype=np.uint64)
    out[: flags.shape[0]] = flags.astype(np.uint64)
    w = out.reshape(words, 32)
    packed = (w << np.arange(32, dtype=np.uint64)).sum(axis=1).astype(np.uint32)
    return packed.view(np.int32)


class LayerCache:
    """A prefilled cache of one layer of workload ``w`` plus its source tensors."""

    def __init__(self, w: W.Workload, layer: int = 0, device="cuda", batch_rows=None,
                 table: Optional[np.ndarray] = None, keep_sources: bool = True,
                 host_pages: int = 0, pool: bool = False, errors: bool = False):
        import torch

        self.w, self.layer, self.device = w, layer, device
        self.pooled = pool
        self.lengths = w.lengths()
        if table is None:
            table, num_pages = W.page_table(w, layer)
        else:
            num_pages = int(table.max()) + 1
        self.table_np = table
        self.max_ctx = w.max_ctx()
        self.table = torch.from_numpy(table).to(device)
        self.seq_lens = torch.from_numpy(self.lengths.astype(np.int32)).to(device)
        self.cache = Cache(w.batch, w.kv_heads, w.head_dim, self.max_ctx, num_pages,
                           self.table, self.seq_lens, device=device, protect=w.protect,
                           host_pages=host_pages,
                           pool_capacity=pool_capacity_for(w) if pool else 0, errors=errors)
        self.num_pages = num_pages
        self.host_free = list(range(num_pages, num_pages + host_pages))  # free host-tier page ids
        self.dev_free = []  # device pages released by demotion
        self.k_src = {}
        self.v_src = {}
        self._prefill(keep_sources)

    # -------------------------------------------------------------- prefill
    def _prefill(self, keep_sources: bool):
        import torch

        w = self.w
        dt = torch.bfloat16 if w.src_dtype == "bf16" else torch.float32
        # prefill in sequence batches so the staging tensor stays small
        lmax = int(self.lengths.max())
        per = max(1, int(2 ** 29 // max(1, lmax * w.kv_heads * w.head_dim * 2)))
        for b0 in range(0, w.batch, per):
            b1 = min(w.batch, b0 + per)
            k_new = torch.zeros((b1 - b0, lmax, w.kv_heads, w.head_dim), dtype=dt, device=self.device)
            v_new = torch.zeros_like(k_new)
            n_new = torch.zeros(b1 - b0, dtype=torch.int32, device=self.device)
            for b in range(b0, b1):
                L = int(self.lengths[b])
                k = W.kv_source_torch(w, self.layer, "K", b, 0, L, self.device)
                v = W.kv_source_torch(w, self.layer, "V", b, 0, L, self.device)
                k_new[b - b0, :L] = k
                v_new[b - b0, :L] = v
                n_new[b - b0] = L
                if keep_sources:
                    self.k_src[b] = k
                    self.v_src[b] = v
            sub = self._sub_cache(b0, b1)
            kvc_quantize_append(sub, k_new, v_new, n_new)
            if w.mask == "mlp":
                self._mlp_subset(sub, k_new, v_new, n_new)
            del k_new, v_new
        self._mask()

    def _sub_cache(self, b0: int, b1: int) -> Cache:
        """A descriptor view of sequences [b0, b1) sharing this cache's memory."""
        if b0 == 0 and b1 == self.w.batch:
            return self.cache
        import copy

        c = self.cache
        sub = copy.copy(c)
        sub.desc = type(c.desc).from_buffer_copy(c.desc)
        D = self.w.head_dim
        sub.desc.batch = b1 - b0
        if c.protect:
            sub.desc.int8_codes = c.int8_codes[b0:b1].data_ptr()
            sub.desc.int8_scales = c.int8_scales[b0:b1].data_ptr()
        sub.desc.block_table = self.table[b0:b1].data_ptr()
        sub.desc.seq_lens = self.seq_lens[b0:b1].data_ptr()
        sub.desc.keep_mask = c.keep_mask[b0:b1].data_ptr()
        sub.desc.scores = c.scores[b0:b1].data_ptr()
        if c.pool is not None:
            sub.desc.pool = c.pool[b0:b1].data_ptr()
            sub.desc.pool_slot = c.pool_slot[b0:b1].data_ptr()
            sub.desc.pool_header = c.pool_header[b0:b1].data_ptr()
        return sub

    def _mlp_subset(self, sub, k_new, v_new, n_new):
        import torch

        if not hasattr(self, "mlp"):
            self.mlp_np = W.mlp_weights(self.w, self.layer)
            self.mlp = torch.from_numpy(self.mlp_np).to(self.device)
        # scores only; the mask is refreshed once for the whole batch afterwards
        kvc_score_topk_mask(sub, self.mlp, k_new, v_new, n_new, 0)

    def _mask(self):
        import torch

        w = self.w
        c = self.cache
        if w.mask == "bernoulli":
            rows = np.zeros((w.batch, w.kv_heads, c.mask_words), dtype=np.int32)
            for b in range(w.batch):
                for h in range(w.kv_heads):
                    L = int(self.lengths[b])
                    rows[b, h] = pack_bits(W.bernoulli_keep_np(w, self.layer, b, h, L), c.mask_words)
            c.keep_mask.copy_(torch.from_numpy(rows))
            if c.pool is not None:
                kvc_pool_build(c)
        elif w.mask == "all":
            kvc_score_topk_mask(c, None, None, None, None, 1000)
        elif w.mask in ("scores", "mlp"):
            if w.mask == "scores":
                for b in range(w.batch):
                    L = int(self.lengths[b])
                    c.scores[b, :, :L] = W.given_scores_torch(w, self.layer, b, L, self.device)
            self.refresh(None, None, None, None)
        else:
            raise ValueError(w.mask)

    def refresh(self, k_new, v_new, n_new, ws=None, stream=None):
        """Score appended tokens (``mlp`` workloads) and refresh the keep mask
        with the workload's policy; ``ws`` is that policy's refresh state or None."""
        w = self.w
        if w.mask == "bernoulli":  # a host-drawn mask; nothing to refresh
            return
        mlp = getattr(self, "mlp", None) if k_new is not None and w.mask == "mlp" else None
        if mlp is None:
            # given scores: a decode step wrote none below the previous lengths, which
            # passing n_new declares (the refresh state may then update in place)
            k_new = v_new = None
        budget = 1000 if w.mask == "all" else w.budget_permille
        if self.block_policy:
            kvc_score_block_mask(self.cache, mlp, k_new, v_new, n_new, budget, w.recency_window,
                                 w.block_tokens, ws=ws, stream=stream)
        else:
            kvc_score_topk_mask(self.cache, mlp, k_new, v_new, n_new, budget, ws=ws, stream=stream)

    def append_refresh(self, k_new, v_new, n_new, ws=None, stream=None):
        """One decode-step update: append the rows, score them and refresh the
        keep mask (one launch for the token policy with MLP scores)."""
        w = self.w
        if w.mask in ("scores", "all") and not self.block_policy:
            # the caller's scores (or keep-all): n_new declares the older ones
            # unchanged, so the encoding and the refresh run as one launch
            budget = 1000 if w.mask == "all" else w.budget_permille
            kvc_append_score_topk_mask(self.cache, None, k_new, v_new, n_new, budget, ws=ws,
                                       stream=stream)
            return
        if w.mask == "mlp" and getattr(self, "mlp", None) is not None:
            if self.block_policy:
                kvc_append_score_block_mask(self.cache, self.mlp, k_new, v_new, n_new,
                                            w.budget_permille, w.recency_window, w.block_tokens,
                                            ws=ws, stream=stream)
            else:
                kvc_append_score_topk_mask(self.cache, self.mlp, k_new, v_new, n_new,
                                           w.budget_permille, ws=ws, stream=stream)
            return
        kvc_quantize_append(self.cache, k_new, v_new, n_new, stream=stream)
        self.refresh(k_new, v_new, n_new, ws=ws, stream=stream)

    @property
    def block_policy(self) -> bool:
        return self.w.policy == "block" and self.w.mask in ("scores", "mlp")

    def refresh_state(self):
        """A zero-filled refresh state for this cache's keep policy."""
        if self.block_policy:
            return block_workspace(self.cache, self.w.block_tokens, self.device)
        return topk_workspace(self.cache, self.device)

    # -------------------------------------------------------------- tiers
    def _move_pages(self, mode: int, free: list) -> int:
        """Find pages (kvc_find_pages ``mode``), copy them to pages from ``free``
        and point the block table at the copies; returns how many moved."""
        import torch

        c = self.cache
        cap = self.w.batch * self.table.shape[1]
        out = torch.empty((cap, 2), dtype=torch.int32, device=self.device)
        count = torch.empty(1, dtype=torch.int32, device=self.device)
        kvc_find_pages(c, mode, out, count)
        n = min(int(count.item()), cap, len(free))
        if n == 0:
            return 0
        sel = out[:n].long()
        src = self.table[sel[:, 0], sel[:, 1]].clone()
        dst = torch.tensor(free[:n], dtype=torch.int32, device=self.device)
        del free[:n]
        kvc_copy_pages(c, src, dst)
        self.table[sel[:, 0], sel[:, 1]] = dst
        return n, src

    def demote_cold_pages(self) -> int:
        """Move device pages whose positions are all evicted to the host tier."""
        r = self._move_pages(0, self.host_free)
        if not r:
            return 0
        n, src = r
        self.dev_free.extend(src.tolist())
        return n

    def promote_hot_pages(self) -> int:
        """Move host-tier pages with a kept position back to released device pages."""
        r = self._move_pages(1, self.dev_free)
        if not r:
            return 0
        n, src = r
        self.host_free.extend(src.tolist())
        return n

    def stream_int4_region(self) -> int:
        """Move every whole page of the INT4 region to the host tier, so that all
        kept INT4 positions are read over the host link."""
        import torch

        ns, nr = (16, 128) if self.w.protect else (0, 0)
        pairs = [(b, lp) for b in range(self.w.batch)
                 for lp in range(ns // 16, max(0, int(self.lengths[b]) - nr) // 16)
                 if int(self.table_np[b, lp]) < self.num_pages]
        pairs = pairs[: len(self.host_free)]
        if not pairs:
            return 0
        idx = torch.tensor(pairs, dtype=torch.long, device=self.device)
        src = self.table[idx[:, 0], idx[:, 1]].clone()
        dst = torch.tensor(self.host_free[: len(pairs)], dtype=torch.int32, device=self.device)
        del self.host_free[: len(pairs)]
        kvc_copy_pages(self.cache, src, dst)
        self.table[idx[:, 0], idx[:, 1]] = dst
        self.dev_free.extend(src.tolist())
        return len(pairs)

    def host_resident_pages(self) -> int:
        t = self.table
        return int(((t >= self.num_pages)).sum().item())

    def replica(self) -> "LayerCache":
        """An independent copy on the device (same contents, own memory)."""
        import copy

        c = self.cache
        r = copy.copy(self)
        r.table = self.table.clone()
        r.seq_lens = self.seq_lens.clone()
        r.cache = Cache(c.batch, c.kv_heads, c.head_dim, c.max_ctx, c.num_phys_pages, r.table,
                        r.seq_lens, device=self.device, protect=c.protect, host_pages=c.host_pages,
                        pool_capacity=c.pool_capacity, errors=c.errors is not None)
        for name in ("int4_codes", "int4_meta", "int8_codes", "int8_scales", "keep_mask", "scores",
                     "int4_codes_host", "int4_meta_host", "pool", "pool_slot", "pool_header"):
            if getattr(c, name) is not None:
                getattr(r.cache, name).copy_(getattr(c, name))
        r.host_free, r.dev_free = list(self.host_free), list(self.dev_free)
        r.k_src, r.v_src = {}, {}
        return r

    # -------------------------------------------------------------- rollout
    def record_rollout(self, steps: int, ws=None):
        """Run ``steps`` decode steps (append one source token per sequence,
        score, refresh the mask with the workload's policy) and record the keep
        mask after each: int32 [B][Hkv][steps][words], row s belonging to query
        position (prompt length + s). Returns the record and the new lengths."""
        import torch

        w = self.w
        c = self.cache
        rec = torch.zeros((w.batch, w.kv_heads, steps, c.mask_words), dtype=torch.int32,
                          device=self.device)
        one = torch.ones(w.batch, dtype=torch.int32, device=self.device)
        lens = self.lengths.copy()
        for s in range(steps):
            k_new = W.kv_rows_torch(w, self.layer, "K", lens, self.device)[:, None]
            v_new = W.kv_rows_torch(w, self.layer, "V", lens, self.device)[:, None]
            lens += 1
            self.seq_lens.add_(1)
            self.append_refresh(k_new, v_new, one, ws=ws)
            rec[:, :, s] = c.keep_mask
        self.lengths = lens
        return rec, lens

    # -------------------------------------------------------------- decode
    def queries(self, step: int = 0):
        return W.queries_torch(self.w, self.layer, step, self.device)

    def workspace(self):
        return attention_workspace(self.cache, self.w.q_heads, self.device)


class DenseLayerCache:
    """A prefilled dense bfloat16 cache of one layer of workload ``w`` (the
    uncompressed baseline), with the same page table and source rows as
    :class:`LayerCache` builds for that workload and layer."""

    def __init__(self, w: W.Workload, layer: int = 0, device="cuda", table: Optional[np.ndarray] = None):
        import torch

        self.w, self.layer, self.device = w, layer, device
        self.lengths = w.lengths()
        if table is None:
            table, num_pages = W.page_table(w, layer)
        else:
            num_pages = int(table.max()) + 1
        self.table_np = table
        self.max_ctx = w.max_ctx()
        self.table = torch.from_numpy(table).to(device)
        self.seq_lens = torch.from_numpy(self.lengths.astype(np.int32)).to(device)
        self.cache = DenseCache(w.batch, w.kv_heads, w.head_dim, self.max_ctx, num_pages,
                                self.table, self.seq_lens, device=device)
        self.num_pages = num_pages
        self._prefill()

    def _prefill(self):
        import torch

        w = self.w
        dt = torch.bfloat16 if w.src_dtype == "bf16" else torch.float32
        lmax = int(self.lengths.max())
        if lmax == 0:
            return
        per = max(1, int(2 ** 29 // max(1, lmax * w.kv_heads * w.head_dim * 2)))
        for b0 in range(0, w.batch, per):
            b1 = min(w.batch, b0 + per)
            k_new = torch.zeros((b1 - b0, lmax, w.kv_heads, w.head_dim), dtype=dt, device=self.device)
            v_new = torch.zeros_like(k_new)
            n_new = torch.zeros(w.batch, dtype=torch.int32, device=self.device)
            for b in range(b0, b1):
                L = int(self.lengths[b])
                k_new[b - b0, :L] = W.kv_source_torch(w, self.layer, "K", b, 0, L, self.device)
                v_new[b - b0, :L] = W.kv_source_torch(w, self.layer, "V", b, 0, L, self.device)
                n_new[b] = L
            sub = self._sub_cache(b0, b1)
            kvc_dense_append(sub, k_new, v_new, n_new[b0:b1])
            del k_new, v_new

    def _sub_cache(self, b0: int, b1: int) -> DenseCache:
        if b0 == 0 and b1 == self.w.batch:
            return self.cache
        import copy

        sub = copy.copy(self.cache)
        sub.desc = type(self.cache.desc).from_buffer_copy(self.cache.desc)
        sub.desc.batch = b1 - b0
        sub.desc.block_table = self.table[b0:b1].data_ptr()
        sub.desc.seq_lens = self.seq_lens[b0:b1].data_ptr()
        return sub

    def replica(self) -> "DenseLayerCache":
        """An independent copy on the device (same contents, own memory)."""
        import copy

        c = self.cache
        r = copy.copy(self)
        r.table = self.table.clone()
        r.seq_lens = self.seq_lens.clone()
        r.cache = DenseCache(c.batch, c.kv_heads, c.head_dim, c.max_ctx, c.num_phys_pages, r.table,
                             r.seq_lens, device=self.device)
        r.cache.kv.copy_(c.kv)
        return r

    def append(self, k_new, v_new, n_new, stream=None):
        kvc_dense_append(self.cache, k_new, v_new, n_new, stream=stream)

    def queries(self, step: int = 0):
        return W.queries_torch(self.w, self.layer, step, self.device)

    def workspace(self):
        return dense_workspace(self.cache, self.w.q_heads, self.device)
