"""Python binding of libkvc: compressed-KV decode attention on MI355X (gfx950).

Argument marshalling only: every step of the path runs in the HIP kernels of
``libkvc.so`` (built in-tree by ``build.py``). PyTorch supplies device memory
and the current stream. Importing works without a GPU; any call raises if the
library has not been built.

The functions mirror the C ABI in ``include/kvc.h``:
``kvc_quantize_append``, ``kvc_score_topk_mask``, ``kvc_append_score_topk_mask``,
``kvc_score_block_mask``, ``kvc_append_score_block_mask``, ``kvc_decode_attention``,
``kvc_attention_workspace_bytes``, ``kvc_topk_workspace_bytes``, ``kvc_pool_build``,
``kvc_pool_bytes``, ``kvc_decode_attention_noalloc``,
``kvc_status_string``, ``kvc_last_error``, ``kvc_abi_version``, and for the dense
bfloat16 baseline ``kvc_dense_append``, ``kvc_dense_decode_attention``,
``kvc_dense_attention_workspace_bytes``.
:class:`Cache` owns the torch tensors of one layer's compressed cache and the
``kvc_cache`` descriptor that points at them; :class:`DenseCache` does the same
for a dense bfloat16 cache (``kvc_dense_cache``).
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libkvc.so")

PAGE = 16
N_SINK = 16
N_RECENT = 128
INT8_SLOTS = N_SINK + N_RECENT
GROUP = 32

KVC_BF16 = 0
KVC_F32 = 1


class KvcError(RuntimeError):
    pass


class KvcCacheStruct(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("max_pages_per_seq", ctypes.c_int32),
        ("num_phys_pages", ctypes.c_int32),
        ("n_sink", ctypes.c_int32),
        ("n_recent", ctypes.c_int32),
        ("group", ctypes.c_int32),
        ("max_ctx", ctypes.c_int32),
        ("int4_codes", ctypes.c_void_p),
        ("int4_meta", ctypes.c_void_p),
        ("int8_codes", ctypes.c_void_p),
        ("int8_scales", ctypes.c_void_p),
        ("block_table", ctypes.c_void_p),
        ("seq_lens", ctypes.c_void_p),
        ("keep_mask", ctypes.c_void_p),
        ("scores", ctypes.c_void_p),
        ("num_host_pages", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
        ("int4_codes_host", ctypes.c_void_p),
        ("int4_meta_host", ctypes.c_void_p),
        ("pool_capacity", ctypes.c_int32),
        ("reserved2", ctypes.c_int32),
        ("pool", ctypes.c_void_p),
        ("pool_slot", ctypes.c_void_p),
        ("pool_header", ctypes.c_void_p),
        ("errors", ctypes.c_void_p),
    ]


# bits of the error word
KVC_ERR_LENGTH = 1
KVC_ERR_PAGE = 2
KVC_ERR_POOL = 4


class KvcDenseCacheStruct(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("max_pages_per_seq", ctypes.c_int32),
        ("num_phys_pages", ctypes.c_int32),
        ("max_ctx", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
        ("kv", ctypes.c_void_p),
        ("block_table", ctypes.c_void_p),
        ("seq_lens", ctypes.c_void_p),
    ]


_lib = None

# exported name -> (restype, argtypes)
_SIGNATURES = {
    "kvc_quantize_append": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                           ctypes.c_int, ctypes.c_int32, ctypes.c_void_p,
                                           ctypes.c_void_p]),
    "kvc_score_topk_mask": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                           ctypes.c_void_p, ctypes.c_int, ctypes.c_int32,
                                           ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p,
                                           ctypes.c_size_t, ctypes.c_void_p]),
    "kvc_append_score_topk_mask": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                                  ctypes.c_void_p, ctypes.c_int, ctypes.c_int32,
                                                  ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p,
                                                  ctypes.c_size_t, ctypes.c_void_p]),
    "kvc_score_block_mask": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                            ctypes.c_void_p, ctypes.c_int, ctypes.c_int32,
                                            ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                            ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t,
                                            ctypes.c_void_p]),
    "kvc_append_score_block_mask": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                            ctypes.c_void_p, ctypes.c_int, ctypes.c_int32,
                                            ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                            ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t,
                                            ctypes.c_void_p]),
    "kvc_block_workspace_bytes": (ctypes.c_size_t, [ctypes.c_void_p, ctypes.c_int32]),
    "kvc_find_pages": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, ctypes.c_int32,
                                      ctypes.c_void_p, ctypes.c_void_p]),
    "kvc_copy_pages": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
                                      ctypes.c_void_p]),
    "kvc_shadow_attention": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                            ctypes.c_int, ctypes.c_int32, ctypes.c_int32,
                                            ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                            ctypes.c_int32, ctypes.c_float, ctypes.c_void_p,
                                            ctypes.c_void_p, ctypes.c_void_p]),
    "kvc_decode_attention": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
                                            ctypes.c_int32, ctypes.c_float, ctypes.c_void_p,
                                            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                            ctypes.c_void_p]),
    "kvc_decode_attention_noalloc": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
                                                    ctypes.c_int32, ctypes.c_float, ctypes.c_void_p,
                                                    ctypes.c_void_p, ctypes.c_void_p]),
    "kvc_decode_attention_windowed": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p,
                                                     ctypes.c_int, ctypes.c_int32, ctypes.c_float,
                                                     ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                                     ctypes.c_size_t, ctypes.c_void_p]),
    "kvc_dense_append": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                        ctypes.c_int, ctypes.c_int32, ctypes.c_void_p,
                                        ctypes.c_void_p]),
    "kvc_dense_decode_attention": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
                                                  ctypes.c_int32, ctypes.c_float, ctypes.c_void_p,
                                                  ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                                  ctypes.c_void_p]),
    "kvc_dense_attention_workspace_bytes": (ctypes.c_size_t, [ctypes.c_void_p, ctypes.c_int32]),
    "kvc_stream_read_probe": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                             ctypes.c_void_p]),
    "kvc_attention_workspace_bytes": (ctypes.c_size_t, [ctypes.c_void_p, ctypes.c_int32]),
    "kvc_pool_build": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p]),
    "kvc_pool_bytes": (ctypes.c_size_t, [ctypes.c_void_p]),
    "kvc_topk_workspace_bytes": (ctypes.c_size_t, [ctypes.c_void_p]),
    "kvc_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "kvc_last_error": (ctypes.c_char_p, []),
    "kvc_abi_version": (ctypes.c_int32, []),
}


def lib():
    """The loaded libkvc (raises KvcError when it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise KvcError(f"{LIB_PATH} is missing: build it with "
                           "`python -m decode_attention_compressed_quantize_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _check(status: int, what: str):
    if status != 0:
        L = lib()
        raise KvcError(f"{what}: {L.kvc_status_string(status).decode()} "
                       f"({L.kvc_last_error().decode()})")


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> int:
    import torch

    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _dtype_code(t) -> int:
    import torch

    if t.dtype == torch.bfloat16:
        return KVC_BF16
    if t.dtype == torch.float32:
        return KVC_F32
    raise KvcError(f"unsupported dtype {t.dtype}")


class Cache:
    """Device tensors of one layer's compressed KV cache plus its descriptor.

    ``block_table`` (int32 [B][max_pages]) and ``seq_lens`` (int32 [B]) are
    device tensors owned by the caller; ``seq_lens`` must hold the lengths
    after any append of the current step. ``protect=False`` builds the
    unprotected (pure KV4) cache: no INT8 side cache, n_sink = n_recent = 0.
    ``pool_capacity`` > 0 (a multiple of 64) adds a kept-record pool of that
    many records per (sequence, kv head); ``errors=True`` adds the error word.
    """

    def __init__(self, batch: int, kv_heads: int, head_dim: int, max_ctx: int,
                 num_phys_pages: int, block_table, seq_lens, device="cuda", with_scores=True,
                 protect: bool = True, host_pages: int = 0, pool_capacity: int = 0,
                 errors: bool = False):
        import torch

        self.batch, self.kv_heads, self.head_dim, self.max_ctx = batch, kv_heads, head_dim, max_ctx
        self.num_phys_pages = num_phys_pages
        dev = torch.device(device)
        D = head_dim
        self.int4_codes = torch.zeros((num_phys_pages, kv_heads, PAGE, 2, D // 2), dtype=torch.uint8, device=dev)
        self.int4_meta = torch.zeros((num_phys_pages, kv_heads, PAGE, 2, D // GROUP, 2), dtype=torch.int16, device=dev)
        self.protect = protect
        self.n_sink, self.n_recent = (N_SINK, N_RECENT) if protect else (0, 0)
        if protect:
            self.int8_codes = torch.zeros((batch, kv_heads, INT8_SLOTS, 2, D), dtype=torch.int8, device=dev)
            self.int8_scales = torch.zeros((batch, kv_heads, INT8_SLOTS, 2), dtype=torch.float32, device=dev)
        else:
            self.int8_codes = self.int8_scales = None
        self.mask_words = (max_ctx + 31) // 32
        self.keep_mask = torch.zeros((batch, kv_heads, self.mask_words), dtype=torch.int32, device=dev)
        self.scores = (torch.zeros((batch, kv_heads, max_ctx), dtype=torch.float32, device=dev)
                       if with_scores else None)
        # optional host tier: pinned host pages [num_phys_pages, num_phys_pages + host_pages)
        self.host_pages = host_pages
        if host_pages > 0:
            self.int4_codes_host = torch.zeros((host_pages, kv_heads, PAGE, 2, D // 2),
                                               dtype=torch.uint8, pin_memory=True)
            self.int4_meta_host = torch.zeros((host_pages, kv_heads, PAGE, 2, D // GROUP, 2),
                                              dtype=torch.int16, pin_memory=True)
        else:
            self.int4_codes_host = self.int4_meta_host = None
        # optional kept-record pool: [B][Hkv][cap/32][40*D] bytes, slot map, headers
        self.pool_capacity = pool_capacity
        if pool_capacity > 0:
            self.pool = torch.zeros((batch, kv_heads, pool_capacity // 32, 40 * D), dtype=torch.uint8,
                                    device=dev)
            self.pool_slot = torch.zeros((batch, kv_heads, max_ctx + pool_capacity), dtype=torch.int32,
                                         device=dev)
            self.pool_header = torch.zeros((batch, kv_heads, 4), dtype=torch.int32, device=dev)
        else:
            self.pool = self.pool_slot = self.pool_header = None
        self.errors = torch.zeros(4, dtype=torch.int32, device=dev) if errors else None
        self.block_table = block_table
        self.seq_lens = seq_lens
        assert block_table.dtype == torch.int32 and seq_lens.dtype == torch.int32
        self.desc = KvcCacheStruct(
            batch, kv_heads, head_dim, PAGE, block_table.shape[1], num_phys_pages,
            self.n_sink, self.n_recent, GROUP, max_ctx,
            _ptr(self.int4_codes), _ptr(self.int4_meta), _ptr(self.int8_codes),
            _ptr(self.int8_scales), _ptr(block_table), _ptr(seq_lens), _ptr(self.keep_mask),
            _ptr(self.scores), host_pages, 0, _ptr(self.int4_codes_host), _ptr(self.int4_meta_host),
            pool_capacity, 0, _ptr(self.pool), _ptr(self.pool_slot), _ptr(self.pool_header),
            _ptr(self.errors))

    def ref(self):
        return ctypes.byref(self.desc)

    def error_bits(self) -> int:
        """The error word (KVC_ERR_* bits); 0 when the cache has none."""
        return 0 if self.errors is None else int(self.errors[0].item())

    def nbytes(self) -> int:
        ts = [self.int4_codes, self.int4_meta, self.int8_codes, self.int8_scales, self.keep_mask,
              self.scores, self.pool, self.pool_slot, self.pool_header]
        ts = [t for t in ts if t is not None]
        return sum(t.numel() * t.element_size() for t in ts)


def kvc_abi_version() -> int:
    return lib().kvc_abi_version()


def kvc_status_string(status: int) -> str:
    return lib().kvc_status_string(status).decode()


def kvc_last_error() -> str:
    return lib().kvc_last_error().decode()


def kvc_attention_workspace_bytes(cache: Cache, num_q_heads: int) -> int:
    return lib().kvc_attention_workspace_bytes(cache.ref(), num_q_heads)


def kvc_topk_workspace_bytes(cache: Cache) -> int:
    return lib().kvc_topk_workspace_bytes(cache.ref())


def kvc_pool_bytes(cache: Cache) -> int:
    return int(lib().kvc_pool_bytes(cache.ref()))


def kvc_pool_build(cache: Cache, stream=None):
    """Rebuild the cache's kept-record pool from its keep mask (masks written by the caller)."""
    _check(lib().kvc_pool_build(cache.ref(), _stream(stream)), "kvc_pool_build")


def kvc_quantize_append(cache: Cache, k_new, v_new, n_new, stream=None):
    """Encode k_new/v_new ([B][n_new_max][Hkv][D], bf16 or fp32) at the tail of each sequence."""
    n_max = k_new.shape[1]
    _check(lib().kvc_quantize_append(cache.ref(), _ptr(k_new), _ptr(v_new), _dtype_code(k_new),
                                     n_max, _ptr(n_new), _stream(stream)), "kvc_quantize_append")


def kvc_score_topk_mask(cache: Cache, mlp, k_new, v_new, n_new, budget_permille: int,
                        ws=None, stream=None):
    """Score appended tokens with the per-head MLP (if ``mlp`` is given) and refresh the keep mask.

    ``ws`` is None or a refresh state from :func:`topk_workspace`, kept by the
    caller for this cache from call to call."""
    n_max = 0 if k_new is None else k_new.shape[1]
    src = KVC_BF16 if k_new is None else _dtype_code(k_new)
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().kvc_score_topk_mask(cache.ref(), _ptr(mlp), _ptr(k_new), _ptr(v_new), src, n_max,
                                     _ptr(n_new), int(budget_permille), _ptr(ws), nbytes,
                                     _stream(stream)), "kvc_score_topk_mask")


def kvc_append_score_topk_mask(cache: Cache, mlp, k_new, v_new, n_new, budget_permille: int,
                               ws=None, stream=None):
    """kvc_quantize_append then kvc_score_topk_mask with the same arguments, in one
    launch when every appended row lands in the protected recent window."""
    n_max = k_new.shape[1]
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().kvc_append_score_topk_mask(cache.ref(), _ptr(mlp), _ptr(k_new), _ptr(v_new),
                                            _dtype_code(k_new), n_max, _ptr(n_new),
                                            int(budget_permille), _ptr(ws), nbytes, _stream(stream)),
           "kvc_append_score_topk_mask")


def kvc_append_score_block_mask(cache: Cache, mlp, k_new, v_new, n_new, budget_permille: int,
                                recency_window: int = 0, block_tokens: int = PAGE, ws=None,
                                stream=None):
    """kvc_quantize_append then kvc_score_block_mask with the same arguments, in one
    launch when every appended row lands in the protected recent window."""
    n_max = k_new.shape[1]
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().kvc_append_score_block_mask(cache.ref(), _ptr(mlp), _ptr(k_new), _ptr(v_new),
                                             _dtype_code(k_new), n_max, _ptr(n_new),
                                             int(budget_permille), int(block_tokens),
                                             int(recency_window), _ptr(ws), nbytes, _stream(stream)),
           "kvc_append_score_block_mask")


def kvc_score_block_mask(cache: Cache, mlp, k_new, v_new, n_new, budget_permille: int,
                         recency_window: int = 0, block_tokens: int = PAGE, ws=None, stream=None):
    """Score appended tokens (if ``mlp`` is given) and refresh the keep mask by whole blocks.

    ``ws`` is None or a refresh state from :func:`block_workspace` for the same
    block size, kept by the caller for this cache from call to call."""
    n_max = 0 if k_new is None else k_new.shape[1]
    src = KVC_BF16 if k_new is None else _dtype_code(k_new)
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().kvc_score_block_mask(cache.ref(), _ptr(mlp), _ptr(k_new), _ptr(v_new), src, n_max,
                                      _ptr(n_new), int(budget_permille), int(block_tokens),
                                      int(recency_window), _ptr(ws), nbytes, _stream(stream)),
           "kvc_score_block_mask")


def kvc_block_workspace_bytes(cache: Cache, block_tokens: int = PAGE) -> int:
    return int(lib().kvc_block_workspace_bytes(cache.ref(), int(block_tokens)))


def kvc_decode_attention(cache: Cache, q, out, lse, ws, softmax_scale: float = 0.0, stream=None):
    """Decode attention of q ([B][Hq][D]) into out (fp32 [B][Hq][D]) and lse (fp32 [B][Hq] or None)."""
    nbytes = ws.numel() * ws.element_size()
    _check(lib().kvc_decode_attention(cache.ref(), _ptr(q), _dtype_code(q), q.shape[1],
                                      float(softmax_scale), _ptr(out), _ptr(lse), _ptr(ws), nbytes,
                                      _stream(stream)), "kvc_decode_attention")


def kvc_decode_attention_noalloc(cache: Cache, q, out, lse, softmax_scale: float = 0.0, stream=None):
    """kvc_decode_attention with the library's own per-GPU scratch instead of a workspace
    (no device allocation; calls that overlap on one GPU race)."""
    _check(lib().kvc_decode_attention_noalloc(cache.ref(), _ptr(q), _dtype_code(q), q.shape[1],
                                              float(softmax_scale), _ptr(out), _ptr(lse),
                                              _stream(stream)), "kvc_decode_attention_noalloc")


NOALLOC_SCRATCH_BYTES = 16 << 20


def kvc_decode_attention_windowed(cache: Cache, int4_window: int, q, out, lse, ws,
                                  softmax_scale: float = 0.0, stream=None):
    """Decode attention reading only the last ``int4_window`` INT4-region positions (0: all)."""
    nbytes = ws.numel() * ws.element_size()
    _check(lib().kvc_decode_attention_windowed(cache.ref(), int(int4_window), _ptr(q), _dtype_code(q),
                                               q.shape[1], float(softmax_scale), _ptr(out), _ptr(lse),
                                               _ptr(ws), nbytes, _stream(stream)),
           "kvc_decode_attention_windowed")


def topk_workspace(cache: Cache, device="cuda"):
    """Allocate a zero-filled top-k refresh state for ``cache`` (see kvc_score_topk_mask)."""
    import torch

    n = kvc_topk_workspace_bytes(cache)
    return torch.zeros(max(n // 4, 1), dtype=torch.int32, device=device)


def kvc_find_pages(cache: Cache, mode: int, out, count, stream=None):
    """List logical pages (sequence, page) into ``out`` (int32 [cap][2]); ``count`` (int32 [1])
    receives how many were found. mode 0: cold device pages, 1: hot host pages."""
    cap = 0 if out is None else out.shape[0]
    _check(lib().kvc_find_pages(cache.ref(), int(mode), _ptr(out), cap, _ptr(count), _stream(stream)),
           "kvc_find_pages")


def kvc_copy_pages(cache: Cache, src, dst, stream=None):
    """Copy physical pages src[i] -> dst[i] (int32 device tensors) of either tier."""
    _check(lib().kvc_copy_pages(cache.ref(), _ptr(src), _ptr(dst), int(src.numel()), _stream(stream)),
           "kvc_copy_pages")


def kvc_shadow_attention(q, k, v, seq_lens, prompt_lens, shadow, out, lse=None,
                         softmax_scale: float = 0.0, stream=None):
    """Learner-side causal attention under recorded shadow rows.

    q [B][T][Hq][D], k and v [B][T][Hkv][D] (bf16), seq_lens and prompt_lens
    int32 [B], shadow int32 [B][Hkv][rows][ceil(T/32)] (row r: the keep mask
    used for query position prompt_len + r), out fp32 [B][T][Hq][D], lse fp32
    [B][T][Hq] or None."""
    B, T, Hq, D = q.shape
    Hkv = k.shape[2]
    rows = 0 if shadow is None else shadow.shape[2]
    if shadow is not None and tuple(shadow.shape[:2]) + (shadow.shape[3],) != (B, Hkv, (T + 31) // 32):
        raise ValueError(f"shadow must be [B][Hkv][rows][{(T + 31) // 32}], got {tuple(shadow.shape)}")
    _check(lib().kvc_shadow_attention(_ptr(q), _ptr(k), _ptr(v), _dtype_code(q), B, T, Hq, Hkv, D,
                                      _ptr(seq_lens), _ptr(prompt_lens), _ptr(shadow), rows,
                                      float(softmax_scale), _ptr(out), _ptr(lse), _stream(stream)),
           "kvc_shadow_attention")


def block_workspace(cache: Cache, block_tokens: int = PAGE, device="cuda"):
    """Allocate a zero-filled block refresh state for ``cache`` (see kvc_score_block_mask)."""
    import torch

    n = kvc_block_workspace_bytes(cache, block_tokens)
    return torch.zeros(max(n // 4, 1), dtype=torch.int32, device=device)


def attention_workspace(cache: Cache, num_q_heads: int, device="cuda"):
    """Allocate a zero-filled workspace of the size kvc_decode_attention needs."""
    import torch

    n = kvc_attention_workspace_bytes(cache, num_q_heads)
    return torch.zeros(max(n // 4, 1), dtype=torch.float32, device=device)


# ---------------------------------------------------------------- dense baseline
class DenseCache:
    """Device tensors of one layer's dense bfloat16 paged cache plus its descriptor.

    ``kv`` is int16 [P][Hkv][16][2][D] holding bfloat16 bits (per token the K
    row then the V row); ``block_table`` and ``seq_lens`` as for :class:`Cache`.
    """

    def __init__(self, batch: int, kv_heads: int, head_dim: int, max_ctx: int,
                 num_phys_pages: int, block_table, seq_lens, device="cuda"):
        import torch

        self.batch, self.kv_heads, self.head_dim, self.max_ctx = batch, kv_heads, head_dim, max_ctx
        self.num_phys_pages = num_phys_pages
        self.kv = torch.zeros((num_phys_pages, kv_heads, PAGE, 2, head_dim), dtype=torch.int16,
                              device=torch.device(device))
        self.block_table = block_table
        self.seq_lens = seq_lens
        assert block_table.dtype == torch.int32 and seq_lens.dtype == torch.int32
        self.desc = KvcDenseCacheStruct(batch, kv_heads, head_dim, PAGE, block_table.shape[1],
                                        num_phys_pages, max_ctx, 0, _ptr(self.kv),
                                        _ptr(block_table), _ptr(seq_lens))

    def ref(self):
        return ctypes.byref(self.desc)

    def nbytes(self) -> int:
        return self.kv.numel() * self.kv.element_size()


def kvc_dense_append(cache: DenseCache, k_new, v_new, n_new, stream=None):
    """Store k_new, v_new ([B][n_new_max][Hkv][D], bf16 or fp32) at each sequence's last
    n_new[b] positions (seq_lens already counting them)."""
    _check(lib().kvc_dense_append(cache.ref(), _ptr(k_new), _ptr(v_new), _dtype_code(k_new),
                                  k_new.shape[1], _ptr(n_new), _stream(stream)), "kvc_dense_append")


def kvc_dense_attention_workspace_bytes(cache: DenseCache, num_q_heads: int) -> int:
    return int(lib().kvc_dense_attention_workspace_bytes(cache.ref(), num_q_heads))


def kvc_dense_decode_attention(cache: DenseCache, q, out, lse, ws, softmax_scale: float = 0.0,
                               stream=None):
    """Decode attention of q ([B][Hq][D]) over every cached position into out and lse."""
    nbytes = ws.numel() * ws.element_size()
    _check(lib().kvc_dense_decode_attention(cache.ref(), _ptr(q), _dtype_code(q), q.shape[1],
                                            float(softmax_scale), _ptr(out), _ptr(lse), _ptr(ws),
                                            nbytes, _stream(stream)), "kvc_dense_decode_attention")


def dense_workspace(cache: DenseCache, num_q_heads: int, device="cuda"):
    """Allocate a workspace of the size kvc_dense_decode_attention needs."""
    import torch

    n = kvc_dense_attention_workspace_bytes(cache, num_q_heads)
    return torch.zeros(max(n // 4, 1), dtype=torch.float32, device=device)


def kvc_stream_read_probe(buf, out, stream=None):
    """Read every byte of ``buf`` once (16-byte loads); XOR-fold its 32-bit words into
    ``out`` (int32 [1], zeroed by the caller). A measurement aid for the read ceiling."""
    _check(lib().kvc_stream_read_probe(_ptr(buf), buf.numel() * buf.element_size(), _ptr(out),
                                       _stream(stream)), "kvc_stream_read_probe")
