/*
 * kvc.h - C ABI of libkvc: decode-step attention over a compressed KV cache
 * on AMD Instinct MI355X (gfx950).
 *
 * The method: the KV4-RL review ("KV4-RL: Unlocking Faster Asynchronous
 * Rollouts for RLVR with INT4 KV Cache Quantization"), section 3, stores the
 * whole context in paged, calibration-free INT4 and protects the first 16
 * positions (attention sinks) and the 128 most recent positions in an INT8
 * side cache; attention processes the two regions independently and joins
 * them with an exact softmax merge, never rebuilding the full cache.
 * Evicted INT4 positions are excluded by a binary keep mask of retained
 * indices (Shadow Mask Distillation page, arXiv 2605.06850, Figure 1
 * caption) chosen per head by score -> sort -> truncate to a budget with a
 * small per-head MLP over the K/V vectors (KVP promo page, arXiv
 * 2602.10238, section "Core mechanism").
 *
 * Numeric rules the pages leave open (fixed by this library):
 *   INT4: per (token, kv head, K or V, group of 32 head_dim entries):
 *         scale = fp16((max-min)/15), min = fp16(min) (RNE, saturated),
 *         code = clamp(rint((x - min) * (1/scale)), 0, 15), scale 0 -> code 0;
 *         value = code*scale + min.
 *   INT8: per (token, kv head, K or V): s = max|x|/127 (fp32),
 *         code = clamp(rint(x * (1/s)), -127, 127), s < FLT_MIN -> code 0;
 *         value = code*s.
 *   All of it in float32 round-to-nearest-even, no fused multiply-add.
 *   Logits are (q . k)*softmax_scale; query head h reads kv head h/(Hq/Hkv).
 *
 * Memory layout (all device memory, owned by the caller; D = head_dim,
 * Hkv = num_kv_heads, P = num_phys_pages, B = batch, page = 16 tokens):
 *   int4_codes  uint8  [P][Hkv][16][2][D/2]   per token: K codes then V codes;
 *               byte j of a K (or V) row holds code 2j in its low nibble and
 *               code 2j+1 in its high nibble.
 *   int4_meta   uint16 [P][Hkv][16][2][D/32][2]  IEEE fp16 bits: per token, the K
 *               groups then the V groups, each as (scale, min).
 *   int8_codes  int8   [B][Hkv][144][2][D]    per slot: K codes then V codes.
 *   int8_scales float  [B][Hkv][144][2]       per slot: (K scale, V scale).
 *               Position t lives in slot t (t < 16) or 16 + (t-16) mod 128.
 *   block_table int32  [B][max_pages_per_seq] logical page -> physical page.
 *   seq_lens    int32  [B]                    current length L_b (after any
 *               append made in the same step); never written by the library.
 *   keep_mask   uint32 [B][Hkv][ceil(max_ctx/32)]  bit t%32 of word t/32 is 1
 *               when position t is retained. Only INT4-region bits
 *               ([16, L-128)) are read by attention; the refresh writes 1 for
 *               the protected positions and 0 at and beyond L.
 *   scores      float  [B][Hkv][max_ctx]      per-position utility score.
 *
 * Regions for a sequence of length L: INT8 = [0, min(L,16)) and
 * [max(16, L-128), L); INT4 = [16, L-128) (empty when L <= 144). INT4 codes
 * are written for every appended position, so a position leaving the
 * 128-window needs no re-encoding: the INT4 region simply grows by one.
 *
 * Pure KV4 (n_sink = n_recent = 0; the unprotected configuration the KV4-RL
 * review, section 3, compares against): there is no INT8 region, int8_codes
 * and int8_scales are neither read nor written (they may be NULL), the INT4
 * region is [0, L), every mask bit below L is a policy decision (nothing is
 * protected), and budgets count all L positions. A sequence whose mask keeps
 * nothing gets out = 0, lse = -inf. Scoring and refresh never run in one
 * launch in this configuration (the appended positions are candidates).
 *
 * Besides the compressed cache, the library holds the uncompressed baseline
 * the pages measure against (a dense bfloat16 paged cache, kvc_dense_cache,
 * with kvc_dense_append and kvc_dense_decode_attention) and a streaming-read
 * probe used as a measurement aid (kvc_stream_read_probe).
 *
 * Kept-record pool (optional; pool_capacity > 0): per (sequence, kv head) a
 * compact copy of the INT4 records of the kept INT4-region positions, so that
 * attention streams exactly the bytes it needs (160 per kept token at D = 128)
 * instead of gathering 128-byte code lines and the shared lines of their
 * per-token meta. The keep mask stays the definition of what is attended; the
 * pool is derived from it and maintained by the calls that write the mask:
 *   pool        uint8 [B][Hkv][pool_capacity/32][40*D]  records in tiles of 32,
 *               in an internal order of bytes (treat as opaque); slots
 *               [0, count) hold the kept records in no particular order.
 *   pool_slot   int32 [B][Hkv][max_ctx + pool_capacity]  two maps: entry
 *               pos < max_ctx holds the slot of kept INT4-region position
 *               pos, entry max_ctx + s the position whose record is in slot
 *               s < count (other entries unspecified).
 *   pool_header int32 [B][Hkv][4]  (count, length, magic, n): the kept count,
 *               the sequence length the pool describes, a validity word, and
 *               a counter that kvc_decode_attention uses during a call (the
 *               workgroups of a (sequence, kv head) that have finished; the
 *               last one merges the partial results and sets it back to 0).
 *               The calls that write the pool set it to 0. Because of that
 *               counter, attention calls on one cache with a pool must not
 *               overlap in time (issue them on one stream, or order them).
 * kvc_score_topk_mask / kvc_append_score_topk_mask update the pool with the
 * mask: a decode step copies at most one record per (sequence, kv head); a
 * full refresh copies the records that enter the kept set, into the slots of
 * those that leave (moving tail records down when the set shrinks), as long as
 * the header is valid and at most 1024 records leave and 1024 enter; otherwise
 * it rebuilds the pool from the mask. That update assumes the pool still holds
 * what the previous call left there. kvc_quantize_append clears the validity
 * word of a (sequence, kv head) whose appended rows reach below n_recent
 * positions short of the length the pool describes (a sequence written
 * afresh, a rollback), so the next refresh rebuilds; a caller that changes INT4 records, the mask or the
 * pool by other means zeroes pool_header (or calls kvc_pool_build).
 * kvc_pool_build rebuilds the pool from the mask for callers that write the
 * mask themselves. kvc_decode_attention reads the
 * pool instead of the mask when pool_capacity > 0, so the pool must describe
 * the current lengths: after an append, refresh (or kvc_pool_build) before
 * attending. pool_capacity (a multiple of 64) must hold the largest kept
 * count, floor(budget_permille * n4 / 1000) at n4 = max_ctx - 144 (- 0 without
 * INT8 protection); the refresh returns KVC_E_SHAPE when the budget could
 * exceed it. The block policy (kvc_score_block_mask, kvc_append_score_block_mask)
 * maintains the pool the same way; its largest kept count is
 * floor(budget_permille * nb / 1000) * block_tokens over the nb candidate
 * blocks (ceil(n4 / block_tokens), or ceil(window / block_tokens) + 1 with a
 * recency window), at most n4. kvc_decode_attention_windowed reads the mask.
 *
 * Error word (optional; errors != NULL): kernels OR KVC_ERR_* bits into
 * errors[0] when they meet device contents they cannot use (a length outside
 * [0, max_ctx], a block-table entry outside the page pools for a position
 * below the length, a pool that does not describe the current length). The
 * affected positions are skipped, so the outputs are unspecified; the word
 * tells the caller so. The library never clears it.
 *
 * Shrinking a length (rolling a sequence back) leaves the INT8 ring slots of
 * the positions that are now the most recent holding the later positions
 * that overwrote them: after lowering seq_lens[b] to L, append again (with
 * kvc_quantize_append or the fused update) the source rows of positions
 * [max(16, L - 128), L) of that sequence before attending, and refresh the
 * mask (a refresh after a shrink is a full one).
 *
 * Conventions: every call is enqueued on the caller's stream and never
 * synchronises; argument errors are returned synchronously; kernels never
 * allocate; the library keeps no state besides a thread-local error string.
 * The cache arrays and the q, out and ws buffers of attention must be 16-byte
 * aligned (device allocations are); a misaligned one gives KVC_E_UNSUPPORTED.
 * Device contents (lengths, table entries) are trusted: out-of-range page ids
 * or lengths are skipped by the kernels rather than dereferenced (and flagged
 * in the error word when there is one), which leaves the affected outputs
 * unspecified. Appended K/V rows must be finite: a NaN entry does not
 * propagate into the stored scale and min (their group min and max ignore
 * it), so the stored codes of such a row are unspecified.
 */
#ifndef KVC_H
#define KVC_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KVC_API __attribute__((visibility("default")))
#define KVC_ABI_VERSION 4

typedef enum {
  KVC_OK = 0,
  KVC_E_NULL = -1,        /* a required pointer is NULL */
  KVC_E_SHAPE = -2,       /* a size is out of range or inconsistent */
  KVC_E_UNSUPPORTED = -3, /* a valid but unsupported configuration */
  KVC_E_WORKSPACE = -4,   /* workspace missing or too small */
  KVC_E_LAUNCH = -5       /* a kernel launch failed */
} kvc_status;

typedef enum { KVC_BF16 = 0, KVC_F32 = 1 } kvc_dtype;

/* One compressed KV cache (one layer). Sizes are host values; pointers are
 * device pointers laid out as described above. */
typedef struct kvc_cache {
  int32_t batch;             /* B >= 1 */
  int32_t num_kv_heads;      /* Hkv >= 1 */
  int32_t head_dim;          /* D: 64 or 128 */
  int32_t page_size;         /* must be 16 */
  int32_t max_pages_per_seq; /* >= ceil(max_ctx/16) */
  int32_t num_phys_pages;    /* P >= 1 */
  int32_t n_sink;            /* 16 with INT8 protection, or 0 (pure KV4, see below) */
  int32_t n_recent;          /* 128 with INT8 protection, or 0 (pure KV4) */
  int32_t group;             /* must be 32 */
  int32_t max_ctx;           /* capacity in positions, >= 1 (attention: <= 2089088) */
  uint8_t* int4_codes;
  uint16_t* int4_meta;
  int8_t* int8_codes;
  float* int8_scales;
  const int32_t* block_table;
  const int32_t* seq_lens;
  uint32_t* keep_mask;
  float* scores;
  /* Optional host tier (temporal tiering, see below): physical pages
   * [P, P + H) live in pinned host memory, addressed like the device pool. */
  int32_t num_host_pages;    /* H >= 0 */
  int32_t reserved;          /* 0 */
  uint8_t* int4_codes_host;  /* [H][Hkv][16][2][D/2], or NULL when H = 0 */
  uint16_t* int4_meta_host;  /* [H][Hkv][16][2][D/32][2], or NULL when H = 0 */
  /* Optional kept-record pool (see above): 0, or records per (sequence, kv
   * head), a multiple of 64; with 0 the three pool pointers are unused. */
  int32_t pool_capacity;
  int32_t reserved2;         /* 0 */
  uint8_t* pool;             /* [B][Hkv][pool_capacity/32][40*D] */
  int32_t* pool_slot;        /* [B][Hkv][max_ctx + pool_capacity] */
  int32_t* pool_header;      /* [B][Hkv][4] */
  uint32_t* errors;          /* device uint32 [1] of KVC_ERR_* bits, or NULL */
} kvc_cache;

/* Bits of the error word (kvc_cache.errors). */
#define KVC_ERR_LENGTH 1u      /* a seq_lens entry outside [0, max_ctx] (clamped) */
#define KVC_ERR_PAGE 2u        /* a block-table entry outside the page pools (skipped) */
#define KVC_ERR_POOL 4u        /* attention found a pool that does not describe the length */

/*
 * kvc_quantize_append - encode appended tokens into the cache.
 * Source: KV4-RL review, section 3 (INT4 for the full context, INT8 side
 * cache for the 16 sink and 128 recent positions).
 *   k_new, v_new : device [B][n_new_max][Hkv][D] of type src (BF16 or F32).
 *   n_new        : device int32 [B]; sequence b appends n_new[b] <= n_new_max
 *                  tokens at positions seq_lens[b]-n_new[b] ... seq_lens[b]-1
 *                  (row j of k_new holds position seq_lens[b]-n_new[b]+j).
 *   Writes INT4 codes and meta for every appended position, and INT8 codes
 *   and scales for appended positions that are sinks (< 16) or lie in the
 *   128-position recent window of the new length; a decode append (n_new=1)
 *   overwrites the ring slot of the position that leaves the window.
 *   n_new_max = 0 is a no-op. Needs int4_codes, int4_meta, int8_codes,
 *   int8_scales, block_table, seq_lens.
 */
KVC_API kvc_status kvc_quantize_append(const kvc_cache* c, const void* k_new, const void* v_new,
                                       kvc_dtype src, int32_t n_new_max, const int32_t* n_new,
                                       hipStream_t stream);

/*
 * kvc_score_topk_mask - score appended tokens and refresh the keep mask.
 * Source: KVP promo page (arXiv 2602.10238), section "Core mechanism" (one MLP
 * per head over K/V, scores ranked and truncated to a budget); Shadow Mask
 * Distillation page, Figure 1 caption (binary mask of retained indices).
 *   mlp          : device float [Hkv][32*2D + 32 + 32 + 1] per head:
 *                  W1 [32][2D] row-major (input = K || V), b1 [32], w2 [32], b2;
 *                  or NULL when the caller already wrote `scores`.
 *   k_new, v_new, src, n_new_max, n_new : as for kvc_quantize_append; used
 *                  only when mlp != NULL (scores for the appended positions
 *                  are w2 . relu(W1 [k||v] + b1) + b2 in float32). With
 *                  mlp == NULL, k_new, v_new, src and n_new_max are ignored and
 *                  n_new may be NULL; a non-NULL n_new declares that the scores
 *                  of positions below the previous call's lengths are unchanged
 *                  (the caller wrote only those of appended positions), which
 *                  allows the in-place update described under ws.
 *   budget_permille : 0..1000. For each (sequence, kv head), with
 *                  n4 = max(0, L-144) and k = floor(budget*n4/1000), keeps the k
 *                  INT4-region positions with the highest score; ties keep the
 *                  lower position; NaN ranks below every number.
 *   ws, ws_bytes : NULL, or refresh state of at least kvc_topk_workspace_bytes(c)
 *                  bytes that the caller keeps for this cache from call to call
 *                  (zero-filled before the first call). With NULL every call
 *                  refreshes the mask from all scores. With a state, a call that
 *                  computes the scores itself (mlp != NULL), or whose n_new
 *                  declares the older scores unchanged, after exactly one
 *                  appended position since the previous call with the same
 *                  budget updates the mask in place; otherwise it refreshes
 *                  fully and rebuilds the state. Either way the mask is the one
 *                  defined above. The state assumes the mask and the scores
 *                  below the previous length were not changed by anyone else.
 */
KVC_API kvc_status kvc_score_topk_mask(const kvc_cache* c, const float* mlp, const void* k_new,
                                       const void* v_new, kvc_dtype src, int32_t n_new_max,
                                       const int32_t* n_new, int32_t budget_permille, void* ws,
                                       size_t ws_bytes, hipStream_t stream);

/*
 * kvc_append_score_topk_mask - one decode-step update of a layer's cache:
 * kvc_quantize_append followed by kvc_score_topk_mask with the same arguments,
 * with the same results, in a single launch when that is possible.
 * Source: KV4-RL review, section 3 (quantize-on-append into the INT4 store and
 * the INT8 side cache) and KVP promo page, section "Core mechanism" (score the
 * new tokens, rank, truncate), steps that one decode step performs in order.
 *   Arguments, ownership and errors as for the two calls. When
 *   1 <= n_new_max <= n_recent, every appended position lies in the protected
 *   recent window, whose codes and scores the refresh does not read, so the
 *   encoding, the scoring (mlp != NULL) and the refresh run as one launch,
 *   provided the refresh may be incremental: mlp != NULL, or mlp == NULL with
 *   n_new != NULL (the caller's scores, those below the previous lengths
 *   unchanged, as for kvc_score_topk_mask); otherwise the two calls run in
 *   order on the stream.
 */
KVC_API kvc_status kvc_append_score_topk_mask(const kvc_cache* c, const float* mlp,
                                              const void* k_new, const void* v_new, kvc_dtype src,
                                              int32_t n_new_max, const int32_t* n_new,
                                              int32_t budget_permille, void* ws, size_t ws_bytes,
                                              hipStream_t stream);

/*
 * kvc_score_block_mask - score appended tokens and refresh the keep mask at
 * block granularity, after an optional recency cut.
 * Source: KVP promo page (arXiv 2602.10238), section "Engineering limits": a
 * paged cache evicts whole blocks, so token scores are averaged per block
 * before ranking, and a coarse recency cut narrows the candidates first.
 *   mlp, k_new, v_new, src, n_new_max, n_new : as for kvc_score_topk_mask.
 *   block_tokens : 16, 32 or 64 (one, two or four pages). Block j covers
 *                  INT4-region offsets [B*j, B*j+B), offset = position - 16.
 *   recency_window : 0, or W > 0: only the last W positions of the INT4 region
 *                  (positions >= max(16, L-128-W)) are candidates; older INT4
 *                  positions are evicted.
 *   budget_permille : with nb blocks holding candidates, keeps
 *                  floor(budget*nb/1000) blocks by the float32 mean of their
 *                  candidate positions' scores (summed in position order),
 *                  highest first; ties keep the lower block; NaN ranks below
 *                  every number. Every candidate position of a kept block is
 *                  kept; protected positions are kept, positions >= L cleared.
 *   Returns KVC_E_UNSUPPORTED for another block size, KVC_E_SHAPE for a budget
 *   outside [0, 1000] or a negative window.
 *   ws, ws_bytes : NULL, or refresh state of at least
 *                  kvc_block_workspace_bytes(c, block_tokens) bytes, 16-byte
 *                  aligned, that the caller keeps for this cache from call to
 *                  call (zero-filled before the first call). It holds each
 *                  block's key, the last threshold and how many keys lie above
 *                  and at it per (sequence, kv head); a call recomputes only the
 *                  keys of blocks whose candidates changed since the length it
 *                  recorded, updates those counts by them, and tries the
 *                  previous threshold before a full selection. A different block size or
 *                  window, or a shorter sequence, rebuilds the state. With NULL
 *                  every call works from all scores. The mask is the one defined
 *                  above either way. The state assumes the scores below the
 *                  previous length minus 128 were not changed by anyone else.
 *   The mask it writes is a valid input for kvc_decode_attention like any other.
 *   With pool_capacity > 0 the kept-record pool is updated with the mask (the
 *   records that leave and enter move in place while at most 1024 of each do
 *   and the pool held the previous kept set; otherwise it is rebuilt, which
 *   copies every kept record: always so for max_ctx above 163,840 positions).
 *   Returns KVC_E_WORKSPACE for a state smaller than required, KVC_E_SHAPE
 *   when the budget could keep more records than pool_capacity holds.
 */
KVC_API kvc_status kvc_score_block_mask(const kvc_cache* c, const float* mlp, const void* k_new,
                                        const void* v_new, kvc_dtype src, int32_t n_new_max,
                                        const int32_t* n_new, int32_t budget_permille,
                                        int32_t block_tokens, int32_t recency_window, void* ws,
                                        size_t ws_bytes, hipStream_t stream);

/*
 * kvc_append_score_block_mask - kvc_quantize_append followed by
 * kvc_score_block_mask with the same arguments, with the same results, in a
 * single launch when that is possible (the block-policy counterpart of
 * kvc_append_score_topk_mask, under the same condition: mlp != NULL and
 * 1 <= n_new_max <= n_recent). Arguments, ownership and errors as for the two
 * calls. Sources as for those two calls.
 */
KVC_API kvc_status kvc_append_score_block_mask(const kvc_cache* c, const float* mlp,
                                               const void* k_new, const void* v_new, kvc_dtype src,
                                               int32_t n_new_max, const int32_t* n_new,
                                               int32_t budget_permille, int32_t block_tokens,
                                               int32_t recency_window, void* ws, size_t ws_bytes,
                                               hipStream_t stream);

/*
 * kvc_decode_attention - one decode query per sequence over the compressed cache.
 * Source: KV4-RL review, section 3 (INT4 and INT8 regions processed
 * independently, outputs combined by an exact softmax merge).
 *   q            : device [B][num_q_heads][D] of type q_dtype (BF16 or F32).
 *   num_q_heads  : Hkv, 2*Hkv or 4*Hkv (query heads per kv head G = 1, 2, 4).
 *   softmax_scale: logit scale; <= 0 selects 1/sqrt(D).
 *   out          : device float [B][num_q_heads][D], softmax-weighted values.
 *   lse          : device float [B][num_q_heads] natural-log log-sum-exp of the
 *                  scaled logits over the attended positions, or NULL.
 *   ws, ws_bytes : device scratch of at least
 *                  kvc_attention_workspace_bytes(c, num_q_heads) bytes for the
 *                  per-chunk partials; its contents on entry do not matter.
 *                  Calls sharing one workspace must not overlap; with a pool,
 *                  neither may calls on one cache (see pool_header).
 *   One launch with a pool (the last workgroup of each (sequence, kv head)
 *   merges its partials); two without (chunks, then the merge).
 *   Attends to the INT8 positions and to the INT4-region positions whose
 *   keep_mask bit is set (with a pool: to the pool's records, which are those
 *   positions when the pool describes the current length). A sequence with
 *   L = 0 yields out = 0, lse = -inf.
 *   Accuracy: logits are float32-accurate for any finite query (the query is
 *   scaled per head by a power of two into fp16's range and, when float32,
 *   split into two fp16 parts; codes enter the matrix instructions exactly);
 *   probabilities enter the P.V product as two fp16 parts. Inputs whose
 *   logits (q . k * softmax_scale) exceed float32's range are unsupported.
 */
KVC_API kvc_status kvc_decode_attention(const kvc_cache* c, const void* q, kvc_dtype q_dtype,
                                        int32_t num_q_heads, float softmax_scale, float* out,
                                        float* lse, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * kvc_decode_attention_windowed - kvc_decode_attention restricted to a
 * recency window of the INT4 region.
 * Source: KVP promo page (arXiv 2602.10238), section "Engineering limits": a
 * coarse recency cut (e.g. to the last 16K positions) before the learned
 * selection; what the cut removes is never read.
 *   int4_window : 0 (the whole region: same as kvc_decode_attention), or W > 0:
 *                 only INT4-region positions in [max(16, L-128-W), L-128) whose
 *                 keep_mask bit is set are attended, plus every INT8 position;
 *                 mask bits of older INT4 positions are not read. Work is
 *                 planned over W positions per sequence instead of max_ctx.
 *   Other arguments, the workspace size and errors as kvc_decode_attention;
 *   KVC_E_SHAPE for a negative window.
 */
KVC_API kvc_status kvc_decode_attention_windowed(const kvc_cache* c, int32_t int4_window,
                                                 const void* q, kvc_dtype q_dtype,
                                                 int32_t num_q_heads, float softmax_scale,
                                                 float* out, float* lse, void* ws, size_t ws_bytes,
                                                 hipStream_t stream);

/*
 * kvc_pool_build - rebuild the kept-record pool from the keep mask.
 * Source: KV4-RL review, section 3 (attention over the paged INT4 store and
 * the INT8 side cache) and the Shadow Mask Distillation page, Figure 1 caption
 * (the mask of retained indices decides what is attended): the pool is a
 * compact copy of the INT4 records the mask keeps, so that attention reads
 * only those.
 *   For every (sequence, kv head): copies the INT4 record (codes and meta) of
 *   each INT4-region position whose keep_mask bit is set into slots
 *   0, 1, ... in position order, writes pool_slot for them and sets
 *   pool_header to (count, seq_lens[b], valid). Needs int4_codes, int4_meta,
 *   block_table, seq_lens, keep_mask and the pool arrays. KVC_E_UNSUPPORTED
 *   without a pool; KVC_E_SHAPE when pool_capacity is not a multiple of 64 or
 *   cannot hold max_ctx - 144 records (the whole INT4 region; the call does
 *   not know a budget). Calls that refresh the mask keep the pool up to date
 *   themselves; this call is for masks written by the caller.
 * kvc_pool_bytes - bytes of the pool array for c->pool_capacity (0 if none).
 */
KVC_API kvc_status kvc_pool_build(const kvc_cache* c, hipStream_t stream);
KVC_API size_t kvc_pool_bytes(const kvc_cache* c);

/*
 * kvc_decode_attention_noalloc - kvc_decode_attention without a workspace
 * argument, for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.
 *   The per-chunk partials go to a scratch array of KVC_NOALLOC_SCRATCH_BYTES
 *   (16 MiB) that the library holds in device memory, one copy per GPU, from
 *   when the library is loaded until the process ends; its address is looked
 *   up on each device's first call (with that device current). The call
 *   allocates nothing and frees nothing.
 *   Arguments, results and errors as kvc_decode_attention (the same kernels
 *   run); KVC_E_WORKSPACE when kvc_attention_workspace_bytes(c, num_q_heads)
 *   exceeds KVC_NOALLOC_SCRATCH_BYTES (the caller then needs
 *   kvc_decode_attention with a workspace of its own). The scratch needs no
 *   clearing: every entry a call reads was written earlier in the same call.
 *   All calls on one GPU share its scratch array, so calls that overlap in
 *   time on one GPU (on different streams, or from different threads) race
 *   and give unspecified results; calls ordered on one stream are safe.
 */
#define KVC_NOALLOC_SCRATCH_BYTES 16777216
KVC_API kvc_status kvc_decode_attention_noalloc(const kvc_cache* c, const void* q,
                                                kvc_dtype q_dtype, int32_t num_q_heads,
                                                float softmax_scale, float* out, float* lse,
                                                hipStream_t stream);

/*
 * Host tier (temporal tiering). Source: TTKV promo page (arXiv 2604.19769),
 * strengths section: a temporal-tiered cache keeps hot data in HBM and cold
 * data in DRAM. Physical page ids [0, P) index the device pool (int4_codes,
 * int4_meta), ids [P, P + H) the host pool (int4_codes_host, int4_meta_host,
 * pinned host memory mapped for device access, same layout). Appends and
 * attention read and write pages of either tier in place, so attention over
 * a host page streams it over the host link. The caller chooses the policy:
 *
 * kvc_find_pages - list logical pages by tier and use, for moving them.
 *   mode 0: device-pool pages whose 16 positions all lie in the INT4 region
 *           ([n_sink, L - n_recent)) and are evicted for every kv head (cold);
 *   mode 1: host-pool pages with at least one kept position (hot again).
 *   out   : device int32 [cap][2] of (sequence, logical page), in no order.
 *   count : device int32, set to the number of pages found (which may exceed
 *           cap; only cap entries are written). Nothing else is modified.
 *
 * kvc_copy_pages - for i < n, copy physical page src[i] to dst[i] (INT4 codes
 *   and meta of every kv head), pages of either tier. src, dst: device int32
 *   [n]; out-of-range ids or src == dst skip the entry. The destinations must
 *   be distinct and none may also be a source. The block table is not
 *   changed: the caller points logical pages at their new physical pages.
 */
KVC_API kvc_status kvc_find_pages(const kvc_cache* c, int32_t mode, int32_t* out, int32_t cap,
                                  int32_t* count, hipStream_t stream);
KVC_API kvc_status kvc_copy_pages(const kvc_cache* c, const int32_t* src, const int32_t* dst,
                                  int32_t n, hipStream_t stream);

/*
 * kvc_shadow_attention - learner-side causal attention under the recorded
 * shadow mask.
 * Source: Shadow Mask Distillation page (arXiv 2605.06850), section 1 and the
 * Figure 1 caption: the binary keep mask M of every sparse rollout step is
 * injected into the learner's causal attention (a time-frozen mask), so the
 * learner's query at a generated position attends to exactly the positions
 * the rollout attended at that step.
 *   q            : device bf16 [B][max_len][num_q_heads][D] (learner queries).
 *   k, v         : device bf16 [B][max_len][num_kv_heads][D] (learner's own
 *                  dense keys and values; quantization is not replayed).
 *   dtype        : must be KVC_BF16. D = head_dim: 64 or 128; G = 1, 2 or 4.
 *   seq_lens     : device int32 [B]: positions [0, L_b) are computed.
 *   prompt_lens  : device int32 [B]: queries at positions below P_b attend
 *                  densely and causally (the rollout's prefill).
 *   shadow       : device uint32 [B][num_kv_heads][shadow_rows][ceil(max_len/32)]:
 *                  row r is the keep mask (bit t%32 of word t/32, protected
 *                  positions included) the rollout used for the query at
 *                  position P_b + r, i.e. the mask at cache length P_b + r + 1;
 *                  bits above the query's position are ignored. A generated
 *                  position with no row (r >= shadow_rows) attends nothing.
 *                  NULL allowed when shadow_rows = 0.
 *   softmax_scale: logit scale; <= 0 selects 1/sqrt(D).
 *   out          : device float [B][max_len][num_q_heads][D]; rows at and beyond
 *                  L_b are not written; a row that attends nothing gets 0.
 *   lse          : device float [B][max_len][num_q_heads] natural-log
 *                  log-sum-exp of the scaled logits (-inf if nothing is
 *                  attended), or NULL.
 *   q, k, v and out must be 16-byte aligned. Needs no workspace.
 */
KVC_API kvc_status kvc_shadow_attention(const void* q, const void* k, const void* v, kvc_dtype dtype,
                                        int32_t batch, int32_t max_len, int32_t num_q_heads,
                                        int32_t num_kv_heads, int32_t head_dim,
                                        const int32_t* seq_lens, const int32_t* prompt_lens,
                                        const uint32_t* shadow, int32_t shadow_rows,
                                        float softmax_scale, float* out, float* lse,
                                        hipStream_t stream);

/*
 * Dense bfloat16 paged cache: the uncompressed baseline.
 * Source: KV4-RL review, section 3 - the INT4 cache's rollout speedups are
 * measured against BF16 rollout, whose KV cache holds every K and V row in
 * bfloat16 and whose decode attention reads every cached position. These
 * calls provide that baseline on the same paging and call shape as the
 * compressed cache, for comparison on one harness.
 *   kv          uint16 [P][Hkv][16][2][D]   bfloat16 bits; per token the K row
 *               then the V row (4*D bytes per token and kv head).
 *   block_table int32  [B][max_pages_per_seq], seq_lens int32 [B]: as in
 *               kvc_cache (seq_lens never written by the library).
 */
typedef struct kvc_dense_cache {
  int32_t batch;             /* B >= 1 */
  int32_t num_kv_heads;      /* Hkv >= 1 */
  int32_t head_dim;          /* D: 64 or 128 */
  int32_t page_size;         /* must be 16 */
  int32_t max_pages_per_seq; /* >= ceil(max_ctx/16) */
  int32_t num_phys_pages;    /* P >= 1 */
  int32_t max_ctx;           /* capacity in positions, >= 1 (attention: <= 2097152) */
  int32_t reserved;          /* 0 */
  uint16_t* kv;
  const int32_t* block_table;
  const int32_t* seq_lens;
} kvc_dense_cache;

/*
 * kvc_dense_append - store appended K/V rows in the dense cache.
 *   k_new, v_new, n_new, n_new_max, src: as kvc_quantize_append (row j of
 *   sequence b is position seq_lens[b]-n_new[b]+j). A float32 row is stored
 *   as its bfloat16 round-to-nearest-even, a bfloat16 row unchanged.
 *   Positions outside [0, max_ctx) and pages whose table entry is outside
 *   [0, P) are skipped. k_new and v_new must be 16-byte aligned.
 */
KVC_API kvc_status kvc_dense_append(const kvc_dense_cache* c, const void* k_new, const void* v_new,
                                    kvc_dtype src, int32_t n_new_max, const int32_t* n_new,
                                    hipStream_t stream);

/*
 * kvc_dense_decode_attention - decode attention over every position of the
 * dense cache.
 *   q, q_dtype, num_q_heads, softmax_scale, out, lse: as kvc_decode_attention
 *   (G = num_q_heads/num_kv_heads in {1, 2, 4}); out[b][h] attends to the
 *   positions [0, seq_lens[b]) of kv head h/G, each read in bfloat16; logits
 *   (q . k)*softmax_scale with a float32 query used at float32 accuracy.
 *   ws, ws_bytes : device scratch of at least
 *                  kvc_dense_attention_workspace_bytes(c, num_q_heads) bytes.
 *   Positions whose page's table entry is outside [0, P) are skipped (not
 *   attended). L = 0 yields out = 0, lse = -inf. kv, q, out and ws must be
 *   16-byte aligned.
 */
KVC_API kvc_status kvc_dense_decode_attention(const kvc_dense_cache* c, const void* q,
                                              kvc_dtype q_dtype, int32_t num_q_heads,
                                              float softmax_scale, float* out, float* lse,
                                              void* ws, size_t ws_bytes, hipStream_t stream);
KVC_API size_t kvc_dense_attention_workspace_bytes(const kvc_dense_cache* c, int32_t num_q_heads);

/*
 * kvc_stream_read_probe - a measurement aid, not a step of the method: read a
 * device buffer once with 16-byte non-temporal loads and XOR every 32-bit word into
 * *out (which the caller zeroes first), so that the attention kernels'
 * bandwidth can also be stated against the read rate this part reaches on a
 * streaming pattern, next to the vendor peak.
 *   buf   : device, 16-byte aligned; bytes: a multiple of 16 (0 is a no-op).
 *   out   : device uint32 (4-byte aligned), receives the XOR fold (exact, checkable).
 */
KVC_API kvc_status kvc_stream_read_probe(const void* buf, size_t bytes, uint32_t* out,
                                         hipStream_t stream);

/* Workspace sizes (host-only, no device work). Return 0 for an invalid cache.
 * kvc_topk_workspace_bytes is the size of the optional refresh state of
 * kvc_score_topk_mask: 1056 bytes per (sequence, kv head).
 * kvc_block_workspace_bytes is the size of the optional refresh state of
 * kvc_score_block_mask (the same for block sizes 16, 32 and 64; 0 for any
 * other): per (sequence, kv head) a 64-byte header plus 4 bytes per 16
 * INT4-region positions of a max_ctx-long sequence, rounded up to 16 bytes.
 * One state may serve calls with different block sizes. */
KVC_API size_t kvc_attention_workspace_bytes(const kvc_cache* c, int32_t num_q_heads);
KVC_API size_t kvc_topk_workspace_bytes(const kvc_cache* c);
KVC_API size_t kvc_block_workspace_bytes(const kvc_cache* c, int32_t block_tokens);

/* Host-only helpers. */
KVC_API const char* kvc_status_string(kvc_status s);
KVC_API const char* kvc_last_error(void);
KVC_API int32_t kvc_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* KVC_H */
