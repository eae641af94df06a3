// Internal declarations shared by the libkvc host layer and its kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "../../include/kvc.h"

namespace kvc {

constexpr int kPage = 16;
// INT8 protection: 16 sink and 128 recent positions (kvc_cache.n_sink and
// n_recent), or none (both 0: every position in INT4). Kernels take the
// values from the descriptor.
constexpr int kSink = 16;
constexpr int kRecent = 128;
constexpr int kGroup = 32;
constexpr int kHidden = 32;

__host__ __device__ inline int mlp_floats(int head_dim) { return kHidden * 2 * head_dim + 2 * kHidden + 1; }
__host__ __device__ inline int mask_words(int max_ctx) { return (max_ctx + 31) / 32; }

// How the INT4 region is cut into split-KV chunks for one attention call.
constexpr int kMaxChunk = 8192;  // positions per chunk workgroup (4 waves x 2048)
constexpr int kMaxParts = 256;   // partials per (sequence, kv head) the merge accepts
struct AttnPlan {
  int chunk;   // positions per INT4 chunk (multiple of 256, 1024 .. kMaxChunk)
  int nsplit;  // INT4 chunks per (sequence, kv head); partial index nsplit is the INT8 region
  int int8_first;  // dispatch order: INT8-region workgroups before (1) or after (0) the chunks
  // Pool mode (the cache has a kept-record pool and the call reads all of it):
  // chunk j of a (sequence, kv head) is the j-th of nsplit equal shares of its
  // pool's record count (the workspace layout is the same as mask mode's).
  int pool;
  // Pool mode with one chunk per pair: the chunk's workgroup also does the
  // INT8 region and writes the output itself (no INT8 workgroups, partials or
  // merge).
  int fuse8;
};

// window > 0: chunks cover only the last `window` INT4-region positions.
// pool: plan the pool mode (only with window == 0 and a pool in the cache).
AttnPlan plan_attention(const kvc_cache& c, int num_q_heads, int window, bool pool = false);

// Attention workspace: partials float [B][Hkv][nsplit + 1][G][2 + D] as
// (m, l, o[0..D-1]) with m in log2 units (chunk j at j, the INT8 region at
// nsplit). No initialisation needed.
inline size_t attention_ws_floats(const kvc_cache& c, int num_q_heads, const AttnPlan& p) {
  return (size_t)c.batch * num_q_heads * (size_t)(p.nsplit + 1) * (size_t)(2 + c.head_dim);
}

hipError_t launch_quantize_append(const kvc_cache& c, const void* k_new, const void* v_new,
                                  kvc_dtype src, int n_new_max, const int32_t* n_new,
                                  hipStream_t s);

hipError_t launch_score(const kvc_cache& c, const float* mlp, const void* k_new, const void* v_new,
                        kvc_dtype src, int n_new_max, const int32_t* n_new, hipStream_t s);

// Keep-mask refresh state of one (sequence, kv head), kept in the caller's
// top-k workspace between calls. Keys are composite: (order key of the score
// << 32) | (0xFFFFFFFF - position), so larger means kept first and no two
// keys are equal. a holds the na smallest kept keys (ascending), b the nb
// largest keys not kept (descending); each list is exact for what it holds.
constexpr int kTopkBuf = 64;
constexpr uint32_t kTopkMagic = 0x4B565431u;
struct TopkState {
  uint32_t magic;  // kTopkMagic when valid
  int32_t len;     // sequence length the mask and lists describe
  int32_t k;       // kept INT4-region positions
  int32_t budget;  // budget_permille used
  int32_t na, nb;
  int32_t pad[2];
  uint64_t a[kTopkBuf];
  uint64_t b[kTopkBuf];
};

hipError_t launch_topk(const kvc_cache& c, int budget_permille, TopkState* state, bool incremental,
                       hipStream_t s);
// Block-granular keep-mask refresh from the scores (whole blocks of 16, 32 or
// 64 tokens, up to kMaxBlocks candidate blocks per sequence).
constexpr int kMaxBlocks = 131072;
// Optional refresh state of one (sequence, kv head): this header, then one
// key per INT4-region block by absolute block index (order key of the block's
// mean score over its candidates when the header was written).
constexpr uint32_t kBlockMagic = 0x4B564231u;
struct BlockStateHeader {
  uint32_t magic;   // kBlockMagic when valid
  int32_t len;      // sequence length the keys and threshold describe
  int32_t block;    // block size
  int32_t window;   // recency window
  int32_t budget;   // budget_permille of thr
  uint32_t thr;     // key of the k-th largest block (when has_thr)
  int32_t has_thr;
  // counts of the stored keys above and equal to thr, valid (has_cnt) when
  // the mask was written as exactly "kept = key >= thr"
  uint32_t gt, eq;
  int32_t has_cnt;
  int32_t pad[6];
};
static_assert(sizeof(BlockStateHeader) == 64, "header size");
// Sized for the smallest block (16 tokens), so that every block size finds
// the headers at the same offsets.
inline size_t block_state_stride(const kvc_cache& c) {
  const int slots = c.n_sink + c.n_recent;
  const int n4 = c.max_ctx > slots ? c.max_ctx - slots : 0;
  const size_t keys = (size_t)(n4 + kPage - 1) / kPage;
  return sizeof(BlockStateHeader) + (keys + 3) / 4 * 16;
}
hipError_t launch_block_topk(const kvc_cache& c, int budget_permille, int block_tokens, int window,
                             void* state, hipStream_t s);
// Scoring and block refresh in one launch; only for n_new_max <= n_recent.
// encode: also the quantize-on-append of the same rows (as launch_quantize_append)
hipError_t launch_score_block(const kvc_cache& c, const float* mlp, const void* k_new,
                              const void* v_new, kvc_dtype src, int n_new_max, const int32_t* n_new,
                              int budget_permille, int block_tokens, int window, void* state,
                              bool encode, hipStream_t s);

// Scoring and refresh in one launch; only for n_new_max <= n_recent.
hipError_t launch_score_topk(const kvc_cache& c, const float* mlp, const void* k_new,
                             const void* v_new, kvc_dtype src, int n_new_max, const int32_t* n_new,
                             int budget_permille, TopkState* state, hipStream_t s);
hipError_t launch_append_score_topk(const kvc_cache& c, const float* mlp, const void* k_new,
                                    const void* v_new, kvc_dtype src, int n_new_max,
                                    const int32_t* n_new, int budget_permille, TopkState* state,
                                    hipStream_t s);

// Host tier: page lists and whole-page copies between the two pools.
hipError_t launch_find_pages(const kvc_cache& c, int mode, int32_t* out, int cap, int32_t* count,
                             hipStream_t s);
hipError_t launch_copy_pages(const kvc_cache& c, const int32_t* src, const int32_t* dst, int n,
                             hipStream_t s);

// Learner-side causal attention under recorded shadow rows (bf16 Q, K, V).
hipError_t launch_shadow_attention(const void* q, const void* k, const void* v, int batch,
                                   int max_len, int num_q_heads, int num_kv_heads, int head_dim,
                                   const int32_t* seq_lens, const int32_t* prompt_lens,
                                   const uint32_t* shadow, int shadow_rows, float softmax_scale,
                                   float* out, float* lse, hipStream_t s);

hipError_t launch_attention(const kvc_cache& c, const void* q, kvc_dtype q_dtype, int num_q_heads,
                            float softmax_scale, float* out, float* lse, float* ws,
                            const AttnPlan& plan, int window, hipStream_t s);

// Exact log-sum-exp merge of `parts_per_pair` partials per (sequence, kv head),
// laid out float [B][Hkv][parts_per_pair][G][2 + D] as (m in log2 units, l, o).
hipError_t launch_merge(const float* parts, int parts_per_pair, int batch, int hkv, int G, int D,
                        float* out, float* lse, hipStream_t s);

// Dense bfloat16 paged cache (the uncompressed baseline).
constexpr int kDenseMaxChunk = 8192;  // positions per chunk workgroup (4 waves x 128 pages)
struct DensePlan {
  int chunk;   // positions per chunk (multiple of 128, <= kDenseMaxChunk)
  int nsplit;  // chunks (= partials) per (sequence, kv head), <= kMaxParts
};
DensePlan plan_dense(const kvc_dense_cache& c);
inline size_t dense_ws_floats(const kvc_dense_cache& c, int num_q_heads, const DensePlan& p) {
  return (size_t)c.batch * num_q_heads * (size_t)p.nsplit * (size_t)(2 + c.head_dim);
}
hipError_t launch_dense_append(const kvc_dense_cache& c, const void* k_new, const void* v_new,
                               kvc_dtype src, int n_new_max, const int32_t* n_new, hipStream_t s);
hipError_t launch_dense_attention(const kvc_dense_cache& c, const void* q, kvc_dtype q_dtype,
                                  int num_q_heads, float softmax_scale, float* out, float* lse,
                                  float* ws, const DensePlan& plan, hipStream_t s);

// Kept-record pool rebuilt from the keep mask (layout in pool_layout.h).
hipError_t launch_pool_build(const kvc_cache& c, hipStream_t s);

// Streaming-read probe (measurement aid): XOR of every 32-bit word into *out.
hipError_t launch_stream_read(const void* buf, size_t bytes, uint32_t* out, hipStream_t s);

}  // namespace kvc
