// libkvc host layer: argument validation, split planning, workspace sizing
// and kernel launches behind the C ABI declared in include/kvc.h.
#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <mutex>
#include <string>

#include "kvc_internal.h"

namespace {

thread_local std::string g_last_error;

kvc_status fail(kvc_status s, const char* msg) {
  g_last_error = msg;
  return s;
}

// Validates the host fields of a cache descriptor and the pointers a call needs.
enum Need : unsigned {
  kNeedInt4 = 1u,
  kNeedInt8 = 2u,
  kNeedMask = 4u,
  kNeedScores = 8u,
};

bool misaligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

kvc_status check_cache(const kvc_cache* c, unsigned need) {
  if (!c) return fail(KVC_E_NULL, "cache descriptor is NULL");
  if (c->batch < 1 || c->num_kv_heads < 1 || c->max_ctx < 1 || c->num_phys_pages < 1)
    return fail(KVC_E_SHAPE, "batch, num_kv_heads, max_ctx and num_phys_pages must be >= 1");
  if (c->head_dim != 64 && c->head_dim != 128)
    return fail(KVC_E_UNSUPPORTED, "head_dim must be 64 or 128");
  if (c->page_size != kvc::kPage) return fail(KVC_E_UNSUPPORTED, "page_size must be 16");
  const bool protect = c->n_sink == kvc::kSink && c->n_recent == kvc::kRecent;
  if (!protect && (c->n_sink != 0 || c->n_recent != 0))
    return fail(KVC_E_UNSUPPORTED, "n_sink/n_recent must be 16/128 (INT8 protection) or 0/0");
  if (c->group != kvc::kGroup) return fail(KVC_E_UNSUPPORTED, "group must be 32");
  if ((long long)c->max_pages_per_seq * kvc::kPage < c->max_ctx)
    return fail(KVC_E_SHAPE, "max_pages_per_seq * 16 must cover max_ctx");
  if (!c->block_table || !c->seq_lens) return fail(KVC_E_NULL, "block_table or seq_lens is NULL");
  if ((need & kNeedInt4) && (!c->int4_codes || !c->int4_meta))
    return fail(KVC_E_NULL, "int4_codes or int4_meta is NULL");
  if ((need & kNeedInt8) && protect && (!c->int8_codes || !c->int8_scales))
    return fail(KVC_E_NULL, "int8_codes or int8_scales is NULL");
  if ((need & kNeedMask) && !c->keep_mask) return fail(KVC_E_NULL, "keep_mask is NULL");
  if ((need & kNeedScores) && !c->scores) return fail(KVC_E_NULL, "scores is NULL");
  if (c->num_host_pages < 0) return fail(KVC_E_SHAPE, "num_host_pages must be >= 0");
  if ((need & kNeedInt4) && c->num_host_pages > 0 && (!c->int4_codes_host || !c->int4_meta_host))
    return fail(KVC_E_NULL, "int4_codes_host or int4_meta_host is NULL with num_host_pages > 0");
  if ((long long)c->num_phys_pages + c->num_host_pages > (long long)0x7FFFFFFF / c->num_kv_heads / kvc::kPage)
    return fail(KVC_E_SHAPE, "too many pages");
  const void* ptrs[] = {c->int4_codes, c->int4_meta, c->int8_codes, c->int8_scales, c->keep_mask,
                        c->scores, c->int4_codes_host, c->int4_meta_host, c->pool, c->pool_header};
  for (const void* q : ptrs)
    if (misaligned(q)) return fail(KVC_E_UNSUPPORTED, "cache arrays must be 16-byte aligned");
  if (c->pool_capacity < 0 || c->pool_capacity % 64)
    return fail(KVC_E_SHAPE, "pool_capacity must be 0 or a positive multiple of 64");
  if (c->pool_capacity > 0) {
    if (!c->pool || !c->pool_slot || !c->pool_header)
      return fail(KVC_E_NULL, "pool, pool_slot or pool_header is NULL with pool_capacity > 0");
    if ((long long)c->pool_capacity * 40 * c->head_dim / 32 > 0x7FFFFFFFLL)
      return fail(KVC_E_SHAPE, "pool_capacity too large");
  }
  if (reinterpret_cast<uintptr_t>(c->errors) & 3u)
    return fail(KVC_E_UNSUPPORTED, "errors must be 4-byte aligned");
  return KVC_OK;
}

// INT4-region positions of a max_ctx-long sequence (the most a pool can need).
long long int4_capacity(const kvc_cache* c) {
  const int slots = c->n_sink + c->n_recent;
  return c->max_ctx > slots ? (long long)c->max_ctx - slots : 0;
}

// A refresh that maintains a pool must not keep more records than it holds.
kvc_status check_pool_budget(const kvc_cache* c, int budget_permille) {
  if (c->pool_capacity <= 0) return KVC_OK;
  if ((long long)budget_permille * int4_capacity(c) / 1000 > c->pool_capacity)
    return fail(KVC_E_SHAPE, "the budget can keep more records than pool_capacity holds");
  return KVC_OK;
}

// The same for the block policy: whole blocks of B tokens are kept (the first
// and the last candidate block can be short), at most floor(budget * nb / 1000)
// of the nb candidate blocks.
kvc_status check_pool_block_budget(const kvc_cache* c, int budget_permille, int block_tokens,
                                   int window) {
  if (c->pool_capacity <= 0) return KVC_OK;
  const long long n4 = int4_capacity(c);
  const long long span = window > 0 && window < n4 ? window : n4;
  const long long nb = (span + block_tokens - 1) / block_tokens + (window > 0 ? 1 : 0);
  long long keep = (long long)budget_permille * nb / 1000 * block_tokens;
  if (keep > n4) keep = n4;
  if (keep > c->pool_capacity)
    return fail(KVC_E_SHAPE, "the budget can keep more records than pool_capacity holds");
  return KVC_OK;
}

kvc_status check_append(const void* k_new, const void* v_new, kvc_dtype src, int n_new_max,
                        const int32_t* n_new) {
  if (n_new_max < 0) return fail(KVC_E_SHAPE, "n_new_max must be >= 0");
  if (src != KVC_BF16 && src != KVC_F32) return fail(KVC_E_UNSUPPORTED, "src must be BF16 or F32");
  if (n_new_max > 0 && (!k_new || !v_new || !n_new))
    return fail(KVC_E_NULL, "k_new, v_new or n_new is NULL");
  return KVC_OK;
}

kvc_status check_dense(const kvc_dense_cache* c) {
  if (!c) return fail(KVC_E_NULL, "dense cache descriptor is NULL");
  if (c->batch < 1 || c->num_kv_heads < 1 || c->max_ctx < 1 || c->num_phys_pages < 1)
    return fail(KVC_E_SHAPE, "batch, num_kv_heads, max_ctx and num_phys_pages must be >= 1");
  if (c->head_dim != 64 && c->head_dim != 128)
    return fail(KVC_E_UNSUPPORTED, "head_dim must be 64 or 128");
  if (c->page_size != kvc::kPage) return fail(KVC_E_UNSUPPORTED, "page_size must be 16");
  if ((long long)c->max_pages_per_seq * kvc::kPage < c->max_ctx)
    return fail(KVC_E_SHAPE, "max_pages_per_seq * 16 must cover max_ctx");
  if (!c->kv || !c->block_table || !c->seq_lens)
    return fail(KVC_E_NULL, "kv, block_table or seq_lens is NULL");
  if (misaligned(c->kv)) return fail(KVC_E_UNSUPPORTED, "kv must be 16-byte aligned");
  return KVC_OK;
}

kvc_status launched(hipError_t e) {
  if (e != hipSuccess) {
    g_last_error = std::string("kernel launch failed: ") + hipGetErrorString(e);
    return KVC_E_LAUNCH;
  }
  return KVC_OK;
}

}  // namespace

namespace kvc {

// Pool mode: chunks per (sequence, kv head) such that the chunk and INT8-region
// workgroups of a call fit one resident round of two workgroups per CU on 256
// CUs when the pairs allow it (fewer, longer chunks pay set-up and epilogue
// less often: measured faster than 2x or 4x as many at 10% and 50% kept),
// one chunk per pair otherwise; a chunk keeps at least 512 records.
constexpr long long kPoolSlots = 512;

AttnPlan plan_attention(const kvc_cache& c, int num_q_heads, int window, bool pool) {
  if (pool) {
    AttnPlan p{};
    const long long pairs = (long long)c.batch * c.num_kv_heads;
    const int prot = c.n_sink + c.n_recent > 0 ? 1 : 0;
    long long j = kPoolSlots / pairs - prot;
    const long long by_size = c.pool_capacity / 512;
    if (j > by_size) j = by_size;
    if (j > kMaxParts - 1) j = kMaxParts - 1;
    if (j < 1) j = 1;
    p.pool = 1;
    p.nsplit = (int)j;
    p.chunk = 0;
    // INT8 regions first when each pair has several chunks (they overlap the
    // chunks' streaming). With one chunk per pair: when all chunks are
    // resident at once, INT8 workgroups could only follow them, so the chunk's
    // workgroup does the INT8 region itself and writes the output (fuse8);
    // with more pairs than that, separate INT8 workgroups after the chunks
    // fill the CUs that short sequences free (measured faster on mixed
    // lengths than fusing).
    p.int8_first = j == 1 ? 0 : 1;
    p.fuse8 = j == 1 && pairs <= kPoolSlots ? 1 : 0;
    return p;
  }
  // attention workgroups resident at once: 2 per CU on 256 CUs (74.8 KB of LDS each)
  constexpr long long kResident = 512;
  constexpr long long kTarget = 384;
  const long long end4 =
      c.max_ctx > c.n_sink + c.n_recent ? (long long)c.max_ctx - c.n_recent : 0;
  long long span = end4;  // positions a sequence's chunks must cover
  if (window > 0 && (long long)window + 64 < span) span = (long long)window + 64;
  const long long pairs = (long long)c.batch * c.num_kv_heads;
  long long chunk = (pairs * span + kTarget - 1) / kTarget;
  const long long fit = (span + kMaxParts - 2) / (kMaxParts - 1);  // nsplit + 1 <= kMaxParts
  if (chunk < fit) chunk = fit;
  chunk = (chunk + 255) / 256 * 256;
  if (chunk < 1024) chunk = 1024;
  if (chunk > kMaxChunk) chunk = kMaxChunk;
  AttnPlan p{};
  p.chunk = (int)chunk;
  p.nsplit = span > 0 ? (int)((span + chunk - 1) / chunk) : 1;
  if (window > 0) {
    // never more partials than the whole-region plan, whose count sizes the workspace
    const AttnPlan full = plan_attention(c, num_q_heads, 0);
    if (p.nsplit > full.nsplit) {
      long long c2 = (span + full.nsplit - 1) / full.nsplit;
      c2 = (c2 + 255) / 256 * 256;
      if (c2 < 1024) c2 = 1024;
      p.chunk = (int)c2;
      p.nsplit = (int)((span + c2 - 1) / c2);
    }
  }
  // INT8 regions first (they run beside the chunks) when the whole grid fits
  // one resident round; otherwise after the chunks, where they fill the slots
  // the first chunks to finish free (before them, as many chunks would wait
  // for a slot and finish late: 128K blocks at 10%, 31.8 -> 31.0 us)
  p.int8_first = pairs * (p.nsplit + 1) <= kResident ? 1 : 0;
  return p;
}

DensePlan plan_dense(const kvc_dense_cache& c) {
  // Chunks of whole 32-token wave tiles (4 waves: multiples of 128), long
  // enough for about two resident workgroups per CU on 256 CUs, and short
  // enough that one wave's pages fit its two registers of page ids.
  constexpr long long kTarget = 512;
  const long long pairs = (long long)c.batch * c.num_kv_heads;
  const long long span = c.max_ctx;
  long long chunk = (pairs * span + kTarget - 1) / kTarget;
  const long long fit = (span + kMaxParts - 1) / kMaxParts;  // nsplit <= kMaxParts
  if (chunk < fit) chunk = fit;
  chunk = (chunk + 127) / 128 * 128;
  if (chunk < 512) chunk = 512;
  if (chunk > kDenseMaxChunk) chunk = kDenseMaxChunk;
  DensePlan p;
  p.chunk = (int)chunk;
  p.nsplit = (int)((span + chunk - 1) / chunk);
  return p;
}

}  // namespace kvc

extern "C" {

KVC_API int32_t kvc_abi_version(void) { return KVC_ABI_VERSION; }

KVC_API const char* kvc_last_error(void) { return g_last_error.c_str(); }

KVC_API const char* kvc_status_string(kvc_status s) {
  switch (s) {
    case KVC_OK: return "ok";
    case KVC_E_NULL: return "null pointer";
    case KVC_E_SHAPE: return "bad shape";
    case KVC_E_UNSUPPORTED: return "unsupported configuration";
    case KVC_E_WORKSPACE: return "workspace too small";
    case KVC_E_LAUNCH: return "kernel launch failed";
  }
  return "unknown status";
}

KVC_API size_t kvc_attention_workspace_bytes(const kvc_cache* c, int32_t num_q_heads) {
  if (check_cache(c, 0) != KVC_OK || num_q_heads < 1 || num_q_heads % c->num_kv_heads) return 0;
  const kvc::AttnPlan p = kvc::plan_attention(*c, num_q_heads, 0);
  size_t n = kvc::attention_ws_floats(*c, num_q_heads, p);
  if (c->pool_capacity > 0) {  // the windowed call still plans by positions
    const size_t np = kvc::attention_ws_floats(*c, num_q_heads, kvc::plan_attention(*c, num_q_heads, 0, true));
    if (np > n) n = np;
  }
  return (n * sizeof(float) + 15) / 16 * 16;
}

KVC_API size_t kvc_pool_bytes(const kvc_cache* c) {
  if (check_cache(c, 0) != KVC_OK || c->pool_capacity <= 0) return 0;
  return (size_t)c->batch * c->num_kv_heads * (size_t)(c->pool_capacity / 32) * 40 * c->head_dim;
}

KVC_API kvc_status kvc_pool_build(const kvc_cache* c, hipStream_t stream) {
  kvc_status st = check_cache(c, kNeedInt4 | kNeedMask);
  if (st != KVC_OK) return st;
  if (c->pool_capacity <= 0) return fail(KVC_E_UNSUPPORTED, "the cache has no pool (pool_capacity = 0)");
  if ((long long)c->batch * c->num_kv_heads > 65535)
    return fail(KVC_E_UNSUPPORTED, "more than 65535 (sequence, kv head) pairs");
  return launched(kvc::launch_pool_build(*c, stream));
}

KVC_API size_t kvc_topk_workspace_bytes(const kvc_cache* c) {
  if (check_cache(c, 0) != KVC_OK) return 0;
  return (size_t)c->batch * c->num_kv_heads * sizeof(kvc::TopkState);
}

KVC_API kvc_status kvc_quantize_append(const kvc_cache* c, const void* k_new, const void* v_new,
                                       kvc_dtype src, int32_t n_new_max, const int32_t* n_new,
                                       hipStream_t stream) {
  kvc_status st = check_cache(c, kNeedInt4 | kNeedInt8);
  if (st != KVC_OK) return st;
  st = check_append(k_new, v_new, src, n_new_max, n_new);
  if (st != KVC_OK) return st;
  if (n_new_max == 0) return KVC_OK;
  return launched(kvc::launch_quantize_append(*c, k_new, v_new, src, n_new_max, n_new, stream));
}

KVC_API kvc_status kvc_score_topk_mask(const kvc_cache* c, const float* mlp, const void* k_new,
                                       const void* v_new, kvc_dtype src, int32_t n_new_max,
                                       const int32_t* n_new, int32_t budget_permille, void* ws,
                                       size_t ws_bytes, hipStream_t stream) {
  kvc_status st = check_cache(c, kNeedMask | kNeedScores | (c && c->pool_capacity > 0 ? kNeedInt4 : 0u));
  if (st != KVC_OK) return st;
  if (budget_permille < 0 || budget_permille > 1000)
    return fail(KVC_E_SHAPE, "budget_permille must be in [0, 1000]");
  st = check_pool_budget(c, budget_permille);
  if (st != KVC_OK) return st;
  if (ws) {
    if (ws_bytes < (size_t)c->batch * c->num_kv_heads * sizeof(kvc::TopkState))
      return fail(KVC_E_WORKSPACE, "top-k workspace too small");
    if (misaligned(ws)) return fail(KVC_E_UNSUPPORTED, "ws must be 16-byte aligned");
  }
  if (mlp) {
    st = check_append(k_new, v_new, src, n_new_max, n_new);
    if (st != KVC_OK) return st;
    if (n_new_max > 0 && n_new_max <= c->n_recent)
      return launched(kvc::launch_score_topk(*c, mlp, k_new, v_new, src, n_new_max, n_new,
                                             budget_permille, static_cast<kvc::TopkState*>(ws),
                                             stream));
    if (n_new_max > 0) {
      st = launched(kvc::launch_score(*c, mlp, k_new, v_new, src, n_new_max, n_new, stream));
      if (st != KVC_OK) return st;
    }
  }
  // The incremental update relies on every score below the previous length
  // being unchanged, which holds when this call writes the new scores itself
  // or when the caller declares it by passing n_new.
  return launched(kvc::launch_topk(*c, budget_permille, static_cast<kvc::TopkState*>(ws),
                                   mlp != nullptr || n_new != nullptr, stream));
}

KVC_API kvc_status kvc_append_score_topk_mask(const kvc_cache* c, const float* mlp,
                                              const void* k_new, const void* v_new, kvc_dtype src,
                                              int32_t n_new_max, const int32_t* n_new,
                                              int32_t budget_permille, void* ws, size_t ws_bytes,
                                              hipStream_t stream) {
  kvc_status st = check_cache(c, kNeedInt4 | kNeedInt8 | kNeedMask | kNeedScores);
  if (st != KVC_OK) return st;
  st = check_append(k_new, v_new, src, n_new_max, n_new);
  if (st != KVC_OK) return st;
  if (budget_permille < 0 || budget_permille > 1000)
    return fail(KVC_E_SHAPE, "budget_permille must be in [0, 1000]");
  st = check_pool_budget(c, budget_permille);
  if (st != KVC_OK) return st;
  if (ws) {
    if (ws_bytes < (size_t)c->batch * c->num_kv_heads * sizeof(kvc::TopkState))
      return fail(KVC_E_WORKSPACE, "top-k workspace too small");
    if (misaligned(ws)) return fail(KVC_E_UNSUPPORTED, "ws must be 16-byte aligned");
  }
  // rows appended in this call sit in the protected recent window: the
  // refresh reads neither their codes nor their scores, so all three run in
  // one launch (the refresh is the incremental kind when this call scores the
  // rows or n_new declares the caller's older scores unchanged); otherwise the
  // two calls run in order
  if ((mlp || n_new) && n_new_max > 0 && n_new_max <= c->n_recent)
    return launched(kvc::launch_append_score_topk(*c, mlp, k_new, v_new, src, n_new_max, n_new,
                                                  budget_permille, static_cast<kvc::TopkState*>(ws),
                                                  stream));
  st = kvc_quantize_append(c, k_new, v_new, src, n_new_max, n_new, stream);
  if (st != KVC_OK) return st;
  return kvc_score_topk_mask(c, mlp, k_new, v_new, src, n_new_max, n_new, budget_permille, ws,
                             ws_bytes, stream);
}

KVC_API size_t kvc_block_workspace_bytes(const kvc_cache* c, int32_t block_tokens) {
  if (check_cache(c, 0) != KVC_OK) return 0;
  if (block_tokens != 16 && block_tokens != 32 && block_tokens != 64) return 0;
  return (size_t)c->batch * c->num_kv_heads * kvc::block_state_stride(*c);
}

KVC_API kvc_status kvc_score_block_mask(const kvc_cache* c, const float* mlp, const void* k_new,
                                        const void* v_new, kvc_dtype src, int32_t n_new_max,
                                        const int32_t* n_new, int32_t budget_permille,
                                        int32_t block_tokens, int32_t recency_window, void* ws,
                                        size_t ws_bytes, hipStream_t stream) {
  kvc_status st = check_cache(c, kNeedMask | kNeedScores | (c && c->pool_capacity > 0 ? kNeedInt4 : 0u));
  if (st != KVC_OK) return st;
  if (budget_permille < 0 || budget_permille > 1000)
    return fail(KVC_E_SHAPE, "budget_permille must be in [0, 1000]");
  if (block_tokens != 16 && block_tokens != 32 && block_tokens != 64)
    return fail(KVC_E_UNSUPPORTED, "block_tokens must be 16, 32 or 64");
  if ((long long)c->max_ctx > (long long)kvc::kMaxBlocks * block_tokens)
    return fail(KVC_E_UNSUPPORTED, "too many blocks per sequence");
  if (recency_window < 0) return fail(KVC_E_SHAPE, "recency_window must be >= 0");
  st = check_pool_block_budget(c, budget_permille, block_tokens, recency_window);
  if (st != KVC_OK) return st;
  if (ws) {
    if (ws_bytes < kvc_block_workspace_bytes(c, block_tokens))
      return fail(KVC_E_WORKSPACE, "block refresh state smaller than kvc_block_workspace_bytes");
    if (misaligned(ws)) return fail(KVC_E_UNSUPPORTED, "block refresh state must be 16-byte aligned");
  }
  if (mlp) {
    st = check_append(k_new, v_new, src, n_new_max, n_new);
    if (st != KVC_OK) return st;
    // rows appended in this call sit in the protected recent window, so the
    // refresh does not read their scores and both run in one launch
    if (n_new_max > 0 && n_new_max <= c->n_recent)
      return launched(kvc::launch_score_block(*c, mlp, k_new, v_new, src, n_new_max, n_new,
                                              budget_permille, block_tokens, recency_window, ws,
                                              false, stream));
    if (n_new_max > 0) {
      st = launched(kvc::launch_score(*c, mlp, k_new, v_new, src, n_new_max, n_new, stream));
      if (st != KVC_OK) return st;
    }
  }
  return launched(
      kvc::launch_block_topk(*c, budget_permille, block_tokens, recency_window, ws, stream));
}

KVC_API kvc_status kvc_append_score_block_mask(const kvc_cache* c, const float* mlp,
                                               const void* k_new, const void* v_new, kvc_dtype src,
                                               int32_t n_new_max, const int32_t* n_new,
                                               int32_t budget_permille, int32_t block_tokens,
                                               int32_t recency_window, void* ws, size_t ws_bytes,
                                               hipStream_t stream) {
  kvc_status st = check_cache(c, kNeedInt4 | kNeedInt8 | kNeedMask | kNeedScores);
  if (st != KVC_OK) return st;
  st = check_append(k_new, v_new, src, n_new_max, n_new);
  if (st != KVC_OK) return st;
  if (budget_permille < 0 || budget_permille > 1000)
    return fail(KVC_E_SHAPE, "budget_permille must be in [0, 1000]");
  if (block_tokens != 16 && block_tokens != 32 && block_tokens != 64)
    return fail(KVC_E_UNSUPPORTED, "block_tokens must be 16, 32 or 64");
  if ((long long)c->max_ctx > (long long)kvc::kMaxBlocks * block_tokens)
    return fail(KVC_E_UNSUPPORTED, "too many blocks per sequence");
  if (recency_window < 0) return fail(KVC_E_SHAPE, "recency_window must be >= 0");
  st = check_pool_block_budget(c, budget_permille, block_tokens, recency_window);
  if (st != KVC_OK) return st;
  if (ws) {
    if (ws_bytes < kvc_block_workspace_bytes(c, block_tokens))
      return fail(KVC_E_WORKSPACE, "block refresh state smaller than kvc_block_workspace_bytes");
    if (misaligned(ws)) return fail(KVC_E_UNSUPPORTED, "block refresh state must be 16-byte aligned");
  }
  // as kvc_append_score_topk_mask: one launch when the rows land in the protected window
  if (mlp && n_new_max > 0 && n_new_max <= c->n_recent)
    return launched(kvc::launch_score_block(*c, mlp, k_new, v_new, src, n_new_max, n_new,
                                            budget_permille, block_tokens, recency_window, ws,
                                            true, stream));
  st = kvc_quantize_append(c, k_new, v_new, src, n_new_max, n_new, stream);
  if (st != KVC_OK) return st;
  return kvc_score_block_mask(c, mlp, k_new, v_new, src, n_new_max, n_new, budget_permille,
                              block_tokens, recency_window, ws, ws_bytes, stream);
}

static kvc_status decode_attention(const kvc_cache* c, int32_t window, const void* q,
                                   kvc_dtype q_dtype, int32_t num_q_heads, float softmax_scale,
                                   float* out, float* lse, void* ws, size_t ws_bytes,
                                   hipStream_t stream) {
  kvc_status st = check_cache(c, kNeedInt4 | kNeedInt8 | kNeedMask);
  if (st != KVC_OK) return st;
  if (!q || !out) return fail(KVC_E_NULL, "q or out is NULL");
  if (misaligned(q) || misaligned(out) || misaligned(ws))
    return fail(KVC_E_UNSUPPORTED, "q, out and ws must be 16-byte aligned");
  if (q_dtype != KVC_BF16 && q_dtype != KVC_F32)
    return fail(KVC_E_UNSUPPORTED, "q_dtype must be BF16 or F32");
  if (num_q_heads < 1 || num_q_heads % c->num_kv_heads)
    return fail(KVC_E_SHAPE, "num_q_heads must be a positive multiple of num_kv_heads");
  const int G = num_q_heads / c->num_kv_heads;
  if (G > 4 || (G & (G - 1)))
    return fail(KVC_E_UNSUPPORTED, "num_q_heads/num_kv_heads must be 1, 2 or 4");
  if ((long long)c->max_ctx > (long long)(kvc::kMaxParts - 1) * kvc::kMaxChunk + c->n_recent)
    return fail(KVC_E_UNSUPPORTED, "max_ctx above (255 * 8192 + n_recent) positions is not supported");
  if (window < 0) return fail(KVC_E_SHAPE, "int4_window must be >= 0");
  const bool pool = c->pool_capacity > 0 && window == 0;
  const size_t need = kvc_attention_workspace_bytes(c, num_q_heads);
  if (!ws || ws_bytes < need) return fail(KVC_E_WORKSPACE, "attention workspace too small");
  const kvc::AttnPlan plan = kvc::plan_attention(*c, num_q_heads, window, pool);
  const float scale = softmax_scale > 0.0f ? softmax_scale : 1.0f / std::sqrt((float)c->head_dim);
  return launched(kvc::launch_attention(*c, q, q_dtype, num_q_heads, scale, out, lse,
                                        static_cast<float*>(ws), plan, window, stream));
}

KVC_API kvc_status kvc_decode_attention(const kvc_cache* c, const void* q, kvc_dtype q_dtype,
                                        int32_t num_q_heads, float softmax_scale, float* out,
                                        float* lse, void* ws, size_t ws_bytes, hipStream_t stream) {
  return decode_attention(c, 0, q, q_dtype, num_q_heads, softmax_scale, out, lse, ws, ws_bytes,
                          stream);
}

// Scratch of the allocation-free attention entry point: one copy per GPU,
// held by the loaded code object until the process ends. Host code never
// uses this name as an address; it uses the per-device pointer that
// hipGetSymbolAddress returned for it.
static __device__ __align__(256) unsigned char scratch[KVC_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// The device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept; NULL on failure.
void* scratch_ptr(kvc_status* st) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    *st = fail(KVC_E_LAUNCH, "no current HIP device (or device index above 63)");
    return nullptr;
  }
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p) return p;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
  if (!p) {
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      g_last_error = std::string("hipGetSymbolAddress of the attention scratch failed: ") +
                     hipGetErrorString(e);
      *st = KVC_E_LAUNCH;
      return nullptr;
    }
    g_scratch_ptr[dev].store(p, std::memory_order_release);
  }
  return p;
}
}  // namespace

KVC_API kvc_status kvc_decode_attention_noalloc(const kvc_cache* c, const void* q,
                                                kvc_dtype q_dtype, int32_t num_q_heads,
                                                float softmax_scale, float* out, float* lse,
                                                hipStream_t stream) {
  kvc_status st = check_cache(c, kNeedInt4 | kNeedInt8 | kNeedMask);
  if (st != KVC_OK) return st;
  const size_t need = kvc_attention_workspace_bytes(c, num_q_heads);
  if (need > (size_t)KVC_NOALLOC_SCRATCH_BYTES) {
    char msg[160];
    std::snprintf(msg, sizeof msg,
                  "this cache needs %zu bytes of attention scratch; the allocation-free entry point "
                  "holds %d bytes (use kvc_decode_attention with a workspace)",
                  need, KVC_NOALLOC_SCRATCH_BYTES);
    return fail(KVC_E_WORKSPACE, msg);
  }
  void* ws = scratch_ptr(&st);
  if (!ws) return st;
  return decode_attention(c, 0, q, q_dtype, num_q_heads, softmax_scale, out, lse, ws,
                          (size_t)KVC_NOALLOC_SCRATCH_BYTES, stream);
}

KVC_API kvc_status kvc_decode_attention_windowed(const kvc_cache* c, int32_t int4_window,
                                                 const void* q, kvc_dtype q_dtype,
                                                 int32_t num_q_heads, float softmax_scale,
                                                 float* out, float* lse, void* ws, size_t ws_bytes,
                                                 hipStream_t stream) {
  return decode_attention(c, int4_window, q, q_dtype, num_q_heads, softmax_scale, out, lse, ws,
                          ws_bytes, stream);
}

KVC_API kvc_status kvc_find_pages(const kvc_cache* c, int32_t mode, int32_t* out, int32_t cap,
                                  int32_t* count, hipStream_t stream) {
  kvc_status st = check_cache(c, kNeedMask);
  if (st != KVC_OK) return st;
  if (mode != 0 && mode != 1) return fail(KVC_E_SHAPE, "mode must be 0 (cold device pages) or 1 (hot host pages)");
  if (!count || (cap > 0 && !out)) return fail(KVC_E_NULL, "out or count is NULL");
  if (cap < 0) return fail(KVC_E_SHAPE, "cap must be >= 0");
  return launched(kvc::launch_find_pages(*c, mode, out, cap, count, stream));
}

KVC_API kvc_status kvc_copy_pages(const kvc_cache* c, const int32_t* src, const int32_t* dst,
                                  int32_t n, hipStream_t stream) {
  kvc_status st = check_cache(c, kNeedInt4);
  if (st != KVC_OK) return st;
  if (n < 0) return fail(KVC_E_SHAPE, "n must be >= 0");
  if (n == 0) return KVC_OK;
  if (!src || !dst) return fail(KVC_E_NULL, "src or dst is NULL");
  return launched(kvc::launch_copy_pages(*c, src, dst, n, stream));
}

KVC_API kvc_status kvc_shadow_attention(const void* q, const void* k, const void* v, kvc_dtype dtype,
                                        int32_t batch, int32_t max_len, int32_t num_q_heads,
                                        int32_t num_kv_heads, int32_t head_dim,
                                        const int32_t* seq_lens, const int32_t* prompt_lens,
                                        const uint32_t* shadow, int32_t shadow_rows,
                                        float softmax_scale, float* out, float* lse,
                                        hipStream_t stream) {
  if (!q || !k || !v || !out || !seq_lens || !prompt_lens)
    return fail(KVC_E_NULL, "q, k, v, out, seq_lens or prompt_lens is NULL");
  if (shadow_rows < 0) return fail(KVC_E_SHAPE, "shadow_rows must be >= 0");
  if (shadow_rows > 0 && !shadow) return fail(KVC_E_NULL, "shadow is NULL");
  if (batch < 1 || max_len < 1 || num_kv_heads < 1 || num_q_heads < 1)
    return fail(KVC_E_SHAPE, "batch, max_len and head counts must be >= 1");
  if (dtype != KVC_BF16) return fail(KVC_E_UNSUPPORTED, "q, k and v must be BF16");
  if (head_dim != 64 && head_dim != 128) return fail(KVC_E_UNSUPPORTED, "head_dim must be 64 or 128");
  if (num_q_heads % num_kv_heads)
    return fail(KVC_E_SHAPE, "num_q_heads must be a multiple of num_kv_heads");
  const int G = num_q_heads / num_kv_heads;
  if (G > 4 || (G & (G - 1)))
    return fail(KVC_E_UNSUPPORTED, "num_q_heads/num_kv_heads must be 1, 2 or 4");
  if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(out))
    return fail(KVC_E_UNSUPPORTED, "q, k, v and out must be 16-byte aligned");
  const float scale = softmax_scale > 0.0f ? softmax_scale : 1.0f / std::sqrt((float)head_dim);
  return launched(kvc::launch_shadow_attention(q, k, v, batch, max_len, num_q_heads, num_kv_heads,
                                               head_dim, seq_lens, prompt_lens, shadow,
                                               shadow_rows, scale, out, lse, stream));
}

KVC_API kvc_status kvc_dense_append(const kvc_dense_cache* c, const void* k_new, const void* v_new,
                                    kvc_dtype src, int32_t n_new_max, const int32_t* n_new,
                                    hipStream_t stream) {
  kvc_status st = check_dense(c);
  if (st != KVC_OK) return st;
  st = check_append(k_new, v_new, src, n_new_max, n_new);
  if (st != KVC_OK) return st;
  if (n_new_max == 0) return KVC_OK;
  if (misaligned(k_new) || misaligned(v_new))
    return fail(KVC_E_UNSUPPORTED, "k_new and v_new must be 16-byte aligned");
  return launched(kvc::launch_dense_append(*c, k_new, v_new, src, n_new_max, n_new, stream));
}

KVC_API size_t kvc_dense_attention_workspace_bytes(const kvc_dense_cache* c, int32_t num_q_heads) {
  if (check_dense(c) != KVC_OK || num_q_heads < 1 || num_q_heads % c->num_kv_heads) return 0;
  return kvc::dense_ws_floats(*c, num_q_heads, kvc::plan_dense(*c)) * sizeof(float);
}

KVC_API kvc_status kvc_dense_decode_attention(const kvc_dense_cache* c, const void* q,
                                              kvc_dtype q_dtype, int32_t num_q_heads,
                                              float softmax_scale, float* out, float* lse,
                                              void* ws, size_t ws_bytes, hipStream_t stream) {
  kvc_status st = check_dense(c);
  if (st != KVC_OK) return st;
  if (!q || !out) return fail(KVC_E_NULL, "q or out is NULL");
  if (misaligned(q) || misaligned(out) || misaligned(ws))
    return fail(KVC_E_UNSUPPORTED, "q, out and ws must be 16-byte aligned");
  if (q_dtype != KVC_BF16 && q_dtype != KVC_F32)
    return fail(KVC_E_UNSUPPORTED, "q_dtype must be BF16 or F32");
  if (num_q_heads < 1 || num_q_heads % c->num_kv_heads)
    return fail(KVC_E_SHAPE, "num_q_heads must be a positive multiple of num_kv_heads");
  const int G = num_q_heads / c->num_kv_heads;
  if (G > 4 || (G & (G - 1)))
    return fail(KVC_E_UNSUPPORTED, "num_q_heads/num_kv_heads must be 1, 2 or 4");
  if ((long long)c->max_ctx > (long long)kvc::kMaxParts * kvc::kDenseMaxChunk)
    return fail(KVC_E_UNSUPPORTED, "max_ctx above 256 * 8192 positions is not supported");
  const kvc::DensePlan plan = kvc::plan_dense(*c);
  const size_t need = kvc::dense_ws_floats(*c, num_q_heads, plan) * sizeof(float);
  if (!ws || ws_bytes < need) return fail(KVC_E_WORKSPACE, "dense attention workspace too small");
  const float scale = softmax_scale > 0.0f ? softmax_scale : 1.0f / std::sqrt((float)c->head_dim);
  return launched(kvc::launch_dense_attention(*c, q, q_dtype, num_q_heads, scale, out, lse,
                                              static_cast<float*>(ws), plan, stream));
}

KVC_API kvc_status kvc_stream_read_probe(const void* buf, size_t bytes, uint32_t* out,
                                         hipStream_t stream) {
  if (bytes == 0) return KVC_OK;
  if (!buf || !out) return fail(KVC_E_NULL, "buf or out is NULL");
  if (misaligned(buf) || bytes % 16) return fail(KVC_E_UNSUPPORTED, "buf must be 16-byte aligned and bytes a multiple of 16");
  if (reinterpret_cast<uintptr_t>(out) & 3u) return fail(KVC_E_UNSUPPORTED, "out must be 4-byte aligned");
  return launched(kvc::launch_stream_read(buf, bytes, out, stream));
}

}  // extern "C"
