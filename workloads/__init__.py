"""Seeded synthetic inputs for compressed-KV decode attention.

This module holds none of the method's arithmetic. It only supplies
counter-based random bits, a fixed table of normal quantiles, and the shapes
of the rollout-style workloads, so that the CPU oracle (tests) and the GPU
path (tests, bench) see identical inputs for the same (stream, index).

Generator: SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom
number generators", OOPSLA 2014; the 64-bit output function of Vigna's
splitmix64). Element ``i`` of a stream with 64-bit key ``k`` is
``mix64(k + (i + 1) * 0x9E3779B97F4A7C15)``. Because every element is a pure
function of its index, a test can regenerate one sequence's slice of a
full-size tensor on the CPU while the GPU generated the whole tensor.

Normal values: the top 16 bits of the output index a table of the 65536
midpoint quantiles of N(0, 1) (``ndtri((i + 0.5) / 65536)`` in float64,
rounded to float32; a bfloat16 copy is the round-to-nearest-even of that).
The distribution is N(0, 1) discretised to 65536 equiprobable levels, which
is finer than bfloat16 resolution over the bulk of the distribution.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Tuple

import numpy as np

MASK64 = (1 << 64) - 1
GAMMA = 0x9E3779B97F4A7C15
M1 = 0xBF58476D1CE4E5B9
M2 = 0x94D049BB133111EB

PAGE = 16            # tokens per physical page
N_SINK = 16          # attention-sink positions held in INT8
N_RECENT = 128       # most recent positions held in INT8
GROUP = 32           # INT4 group along head_dim
MLP_HIDDEN = 32


def _mix64_int(z: int) -> int:
    z &= MASK64
    z = ((z ^ (z >> 30)) * M1) & MASK64
    z = ((z ^ (z >> 27)) * M2) & MASK64
    return z ^ (z >> 31)


def stream_key(*parts) -> int:
    """64-bit stream key from a tuple of names/ints (FNV-1a, then mix64)."""
    h = 0xCBF29CE484222325
    for byte in repr(tuple(parts)).encode():
        h ^= byte
        h = (h * 0x100000001B3) & MASK64
    return _mix64_int(h)


# --------------------------------------------------------------------------
# numpy backend
# --------------------------------------------------------------------------
def bits_np(key: int, idx: np.ndarray) -> np.ndarray:
    """SplitMix64 outputs (uint64) for element indices ``idx`` of stream ``key``."""
    idx = np.asarray(idx, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = np.uint64(key) + (idx + np.uint64(1)) * np.uint64(GAMMA)
        z = (z ^ (z >> np.uint64(30))) * np.uint64(M1)
        z = (z ^ (z >> np.uint64(27))) * np.uint64(M2)
        z = z ^ (z >> np.uint64(31))
    return z


def _make_tables():
    from scipy.special import ndtri

    p = (np.arange(65536, dtype=np.float64) + 0.5) / 65536.0
    t32 = ndtri(p).astype(np.float32)
    b = t32.view(np.uint32).astype(np.uint64)
    bias = ((b >> np.uint64(16)) & np.uint64(1)) + np.uint64(0x7FFF)
    t16 = ((b + bias) >> np.uint64(16)).astype(np.uint16)
    return t32, t16


NORMAL_F32, NORMAL_BF16_BITS = _make_tables()


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns (uint16) to float32."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal_np(key: int, idx: np.ndarray, dtype: str) -> np.ndarray:
    """N(0,1) draws: float32 values (dtype='f32') or bfloat16 bits (dtype='bf16')."""
    top = (bits_np(key, idx) >> np.uint64(48)).astype(np.int64)
    if dtype == "f32":
        return NORMAL_F32[top]
    if dtype == "bf16":
        return NORMAL_BF16_BITS[top]
    raise ValueError(dtype)


def uniform_np(key: int, idx: np.ndarray) -> np.ndarray:
    """U[0,1) float64 draws (53 random bits)."""
    return (bits_np(key, idx) >> np.uint64(11)).astype(np.float64) * (2.0 ** -53)


# --------------------------------------------------------------------------
# torch backend (same bits; int64 arithmetic wraps modulo 2**64)
# --------------------------------------------------------------------------
def _s64(c: int) -> int:
    c &= MASK64
    return c - (1 << 64) if c >= (1 << 63) else c


def _srl(z, s: int):
    return (z >> s) & ((1 << (64 - s)) - 1)


def bits_torch(key: int, idx):
    """SplitMix64 outputs as int64 tensors (two's-complement view of uint64)."""
    z = (idx + 1) * _s64(GAMMA) + _s64(key)
    z = (z ^ _srl(z, 30)) * _s64(M1)
    z = (z ^ _srl(z, 27)) * _s64(M2)
    return z ^ _srl(z, 31)


_TORCH_TABLES = {}


def _torch_tables(device):
    import torch

    dev = torch.device(device)
    if dev not in _TORCH_TABLES:
        _TORCH_TABLES[dev] = (
            torch.from_numpy(NORMAL_F32.copy()).to(dev),
            torch.from_numpy(NORMAL_BF16_BITS.view(np.int16).copy()).to(dev),
        )
    return _TORCH_TABLES[dev]


def normal_torch(key: int, idx, dtype: str):
    """Same draws as :func:`normal_np`; bf16 is returned as a bfloat16 tensor."""
    import torch

    t32, t16 = _torch_tables(idx.device)
    top = _srl(bits_torch(key, idx), 48)
    if dtype == "f32":
        return t32[top]
    if dtype == "bf16":
        return t16[top].view(torch.bfloat16)
    raise ValueError(dtype)


# --------------------------------------------------------------------------
# workloads
# --------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape and input recipe of one synthetic decode workload."""

    name: str
    batch: int
    q_heads: int
    kv_heads: int
    head_dim: int
    layers: int = 1
    ctx: Optional[int] = None                  # uniform context length
    ctx_range: Optional[Tuple[int, int]] = None  # log-uniform per-sequence lengths
    ctx_list: Optional[Tuple[int, ...]] = None   # explicit per-sequence lengths
    src_dtype: str = "bf16"                    # K/V/Q source type: "bf16" or "f32"
    mask: str = "all"                          # "all" | "bernoulli" | "scores" | "mlp"
    budget_permille: Optional[int] = None
    policy: str = "token"                      # keep policy: "token" top-k or "block" (whole blocks)
    block_tokens: int = 16                     # block size of the "block" policy
    recency_window: int = 0                    # "block" policy: candidates = last W INT4 positions (0 = all)
    protect: bool = True                       # INT8 sink/recent protection (False: pure KV4)
    outlier_channels: int = 0                  # (kv head, dim) channels scaled x8
    shuffled_pages: bool = True
    decode_steps: int = 0                      # extra capacity for appended tokens
    seed: int = 0

    @property
    def group_size(self) -> int:
        return self.q_heads // self.kv_heads

    def lengths(self) -> np.ndarray:
        """Per-sequence context lengths (int32 [B])."""
        if self.ctx_list is not None:
            return np.array(self.ctx_list, dtype=np.int32)
        if self.ctx is not None:
            return np.full(self.batch, self.ctx, dtype=np.int32)
        lo, hi = self.ctx_range
        u = uniform_np(stream_key(self.seed, self.name, "len"), np.arange(self.batch))
        ratio = hi / lo
        return np.rint(lo * ratio ** u).astype(np.int32)

    def capacity(self) -> np.ndarray:
        return self.lengths() + self.decode_steps

    def max_ctx(self) -> int:
        return int(self.capacity().max())

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    # Tiny reference case: fp32 sources, Bernoulli(0.5) keep mask on the INT4 region.
    "tiny": Workload("tiny", 1, 4, 1, 64, ctx=512, src_dtype="f32", mask="bernoulli",
                     shuffled_pages=False),
    # Uniform decode, no eviction, 1% outlier channels x8.
    "uniform4k": Workload("uniform4k", 64, 32, 8, 128, ctx=4096, mask="all",
                          outlier_channels=10),
    # Async-rollout long tail: lengths log-uniform in [1K, 16K], given N(0,1) scores, top 50%.
    "longtail": Workload("longtail", 256, 32, 8, 128, ctx_range=(1024, 16384), mask="scores",
                         budget_permille=500),
    # Long context, per-head MLP scores, top-k at 10% and 50%.
    "long128k_b10": Workload("long128k_b10", 4, 32, 8, 128, ctx=131072, mask="mlp",
                             budget_permille=100),
    "long128k_b50": Workload("long128k_b50", 4, 32, 8, 128, ctx=131072, mask="mlp",
                             budget_permille=500),
    # Long context, whole 16-token blocks ranked by mean MLP score, at 10% and 50%.
    "long128k_blk_b10": Workload("long128k_blk_b10", 4, 32, 8, 128, ctx=131072, mask="mlp",
                                 budget_permille=100, policy="block"),
    "long128k_blk_b50": Workload("long128k_blk_b50", 4, 32, 8, 128, ctx=131072, mask="mlp",
                                 budget_permille=500, policy="block"),
    # Long context, coarse recency cut to the last 16K positions, then blocks at 10% / 50%.
    "long128k_r16k_b10": Workload("long128k_r16k_b10", 4, 32, 8, 128, ctx=131072, mask="mlp",
                                  budget_permille=100, policy="block", recency_window=16384),
    "long128k_r16k_b50": Workload("long128k_r16k_b50", 4, 32, 8, 128, ctx=131072, mask="mlp",
                                  budget_permille=500, policy="block", recency_window=16384),
    # The 128K top-k workloads without INT8 protection (pure KV4: every position INT4).
    "long128k_kv4_b10": Workload("long128k_kv4_b10", 4, 32, 8, 128, ctx=131072, mask="mlp",
                                 budget_permille=100, protect=False),
    "long128k_kv4_b50": Workload("long128k_kv4_b50", 4, 32, 8, 128, ctx=131072, mask="mlp",
                                 budget_permille=500, protect=False),
    # Full decode step: 36 layers, append + score + top-k refresh (30%) + attention.
    "fullstep": Workload("fullstep", 128, 32, 8, 128, layers=36, ctx=32768, mask="mlp",
                         budget_permille=300, decode_steps=64),
}


def outlier_set(w: Workload, which: str) -> np.ndarray:
    """Flat indices (kvh * D + d) of the channels scaled x8 for K or V."""
    n = w.outlier_channels
    if n == 0:
        return np.zeros(0, dtype=np.int64)
    cand = w.kv_heads * w.head_dim
    b = bits_np(stream_key(w.seed, w.name, "outlier", which), np.arange(cand))
    return np.sort(np.argsort(b, kind="stable")[:n]).astype(np.int64)


def _kv_key(w: Workload, layer: int, which: str, b: int) -> int:
    return stream_key(w.seed, w.name, which, layer, b)


def kv_source_np(w: Workload, layer: int, which: str, b: int, t0: int, t1: int,
                 kvh: Optional[int] = None) -> np.ndarray:
    """Source K or V of sequence ``b`` for positions [t0, t1).

    Returns bf16 bits (uint16) or float32, shape [t1-t0][Hkv][D], or [t1-t0][D]
    when ``kvh`` is given. Element (t, h, d) is stream index (t*Hkv + h)*D + d.
    """
    H, D = w.kv_heads, w.head_dim
    t = np.arange(t0, t1, dtype=np.int64)
    heads = np.arange(H, dtype=np.int64) if kvh is None else np.array([kvh], dtype=np.int64)
    d = np.arange(D, dtype=np.int64)
    idx = (t[:, None, None] * H + heads[None, :, None]) * D + d[None, None, :]
    x = normal_np(_kv_key(w, layer, which, b), idx.reshape(-1), w.src_dtype).reshape(idx.shape)
    out = outlier_set(w, which)
    if out.size:
        chan = heads[:, None] * D + d[None, :]
        hit = np.isin(chan, out)
        if hit.any():
            if w.src_dtype == "bf16":
                f = bf16_bits_to_f32(x) * np.float32(8.0)
                x = np.where(hit[None], (f.view(np.uint32) >> np.uint32(16)).astype(np.uint16), x)
            else:
                x = np.where(hit[None], x * np.float32(8.0), x)
    return x[:, 0, :] if kvh is not None else x


def kv_source_torch(w: Workload, layer: int, which: str, b: int, t0: int, t1: int, device):
    """Torch twin of :func:`kv_source_np` for all kv heads: [t1-t0][Hkv][D] on ``device``."""
    import torch

    H, D = w.kv_heads, w.head_dim
    n = (t1 - t0) * H * D
    idx = torch.arange(n, dtype=torch.int64, device=device) + t0 * H * D
    x = normal_torch(_kv_key(w, layer, which, b), idx, w.src_dtype).view(t1 - t0, H, D)
    out = outlier_set(w, which)
    if out.size:
        x = x.clone()
        flat = x.view(t1 - t0, H * D)
        sel = torch.from_numpy(out).to(device)
        flat[:, sel] = flat[:, sel] * 8
    return x


def kv_rows_torch(w: Workload, layer: int, which: str, positions, device):
    """One source row per sequence: position ``positions[b]`` of sequence b, [B][Hkv][D].

    Identical values to :func:`kv_source_torch` / :func:`kv_source_np` at those
    positions (the per-sequence stream key enters as a tensor).
    """
    import torch

    H, D = w.kv_heads, w.head_dim
    keys = torch.tensor([_s64(_kv_key(w, layer, which, b)) for b in range(len(positions))],
                        dtype=torch.int64, device=device)
    pos = torch.as_tensor(np.asarray(positions, dtype=np.int64), device=device)
    hd = torch.arange(H * D, dtype=torch.int64, device=device)
    idx = pos[:, None] * (H * D) + hd[None, :]
    z = (idx + 1) * _s64(GAMMA) + keys[:, None]
    z = (z ^ _srl(z, 30)) * _s64(M1)
    z = (z ^ _srl(z, 27)) * _s64(M2)
    z = z ^ _srl(z, 31)
    t32, t16 = _torch_tables(device)
    top = _srl(z, 48)
    x = (t16[top].view(torch.bfloat16) if w.src_dtype == "bf16" else t32[top])
    out = outlier_set(w, which)
    if out.size:
        sel = torch.from_numpy(out).to(device)
        x[:, sel] = x[:, sel] * 8
    return x.view(len(positions), H, D)


def queries_np(w: Workload, layer: int, step: int) -> np.ndarray:
    """Decode queries [B][Hq][D] (bf16 bits or float32)."""
    idx = np.arange(w.batch * w.q_heads * w.head_dim, dtype=np.int64)
    x = normal_np(stream_key(w.seed, w.name, "Q", layer, step), idx, w.src_dtype)
    return x.reshape(w.batch, w.q_heads, w.head_dim)


def queries_torch(w: Workload, layer: int, step: int, device):
    import torch

    n = w.batch * w.q_heads * w.head_dim
    idx = torch.arange(n, dtype=torch.int64, device=device)
    x = normal_torch(stream_key(w.seed, w.name, "Q", layer, step), idx, w.src_dtype)
    return x.view(w.batch, w.q_heads, w.head_dim)


def learner_queries_np(w: Workload, layer: int, b: int, t0: int, t1: int) -> np.ndarray:
    """Learner-side queries of sequence ``b`` for positions [t0, t1): [t1-t0][Hq][D]
    (bf16 bits or float32); element (t, h, d) is stream index (t*Hq + h)*D + d."""
    Hq, D = w.q_heads, w.head_dim
    idx = np.arange(t0 * Hq * D, t1 * Hq * D, dtype=np.int64)
    x = normal_np(stream_key(w.seed, w.name, "LQ", layer, b), idx, w.src_dtype)
    return x.reshape(t1 - t0, Hq, D)


def learner_queries_torch(w: Workload, layer: int, b: int, t0: int, t1: int, device):
    """Torch twin of :func:`learner_queries_np`."""
    import torch

    Hq, D = w.q_heads, w.head_dim
    idx = torch.arange(t0 * Hq * D, t1 * Hq * D, dtype=torch.int64, device=device)
    x = normal_torch(stream_key(w.seed, w.name, "LQ", layer, b), idx, w.src_dtype)
    return x.view(t1 - t0, Hq, D)


def given_scores_np(w: Workload, layer: int, b: int, length: int) -> np.ndarray:
    """Caller-provided per-token scores ~ N(0,1), float32 [Hkv][length]."""
    idx = np.arange(w.kv_heads * length, dtype=np.int64)
    x = normal_np(stream_key(w.seed, w.name, "S", layer, b), idx, "f32")
    return x.reshape(w.kv_heads, length)


def given_scores_torch(w: Workload, layer: int, b: int, length: int, device):
    import torch

    idx = torch.arange(w.kv_heads * length, dtype=torch.int64, device=device)
    return normal_torch(stream_key(w.seed, w.name, "S", layer, b), idx, "f32").view(
        w.kv_heads, length)


def mlp_weights(w: Workload, layer: int) -> np.ndarray:
    """Seeded per-kv-head scorer weights, float32 [Hkv][8257].

    Per head: W1 [32][2D] ~ N(0, 1/(2D)), b1 = 0 [32], w2 [32] ~ N(0, 1/32), b2 = 0.
    """
    D2 = 2 * w.head_dim
    n_w1 = MLP_HIDDEN * D2
    per = n_w1 + 2 * MLP_HIDDEN + 1
    out = np.zeros((w.kv_heads, per), dtype=np.float32)
    for h in range(w.kv_heads):
        w1 = normal_np(stream_key(w.seed, w.name, "W1", layer, h), np.arange(n_w1), "f32")
        w2 = normal_np(stream_key(w.seed, w.name, "W2", layer, h), np.arange(MLP_HIDDEN), "f32")
        out[h, :n_w1] = w1 * np.float32(1.0 / math.sqrt(D2))
        out[h, n_w1 + MLP_HIDDEN: n_w1 + 2 * MLP_HIDDEN] = w2 * np.float32(1.0 / math.sqrt(MLP_HIDDEN))
    return out


def bernoulli_keep_np(w: Workload, layer: int, b: int, kvh: int, length: int) -> np.ndarray:
    """Bernoulli(0.5) keep flags for positions [0, length) (bool)."""
    z = bits_np(stream_key(w.seed, w.name, "keep", layer, b, kvh), np.arange(length))
    return (z >> np.uint64(63)).astype(bool)


def page_table(w: Workload, layer: int = 0):
    """Block table int32 [B][max_pages] and the number of physical pages.

    Each sequence gets ceil(capacity/16) pages. With ``shuffled_pages`` the
    physical page ids are a seeded permutation of all pages; otherwise pages
    are handed out in order.
    """
    cap = w.capacity()
    npages = np.maximum((cap + PAGE - 1) // PAGE, 1)
    total = int(npages.sum())
    max_pages = int(npages.max())
    if w.shuffled_pages:
        z = bits_np(stream_key(w.seed, w.name, "pages", layer), np.arange(total))
        perm = np.argsort(z, kind="stable").astype(np.int32)
    else:
        perm = np.arange(total, dtype=np.int32)
    table = np.full((w.batch, max_pages), -1, dtype=np.int32)
    off = 0
    for b in range(w.batch):
        table[b, : npages[b]] = perm[off: off + npages[b]]
        off += npages[b]
    return table, total
