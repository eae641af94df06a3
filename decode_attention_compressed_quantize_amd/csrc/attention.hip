// Split-region decode attention over the compressed cache, with the exact
// log-sum-exp merge of the per-chunk partials in a second, small launch.
//
// Source: KV4-RL review, section 3 - the INT4 region and the protected INT8
// region are processed independently and their outputs are combined by an
// exact softmax merge, so the full-precision cache is never rebuilt; the
// protected region uses high-fidelity probability-value arithmetic, read here
// as float32 P and float32 decoded V.
//
// Work decomposition: one workgroup (4 waves) per (sequence, kv head, INT4
// chunk of `chunk` positions), plus one workgroup per (sequence, kv head) for
// the INT8 region. Every workgroup writes one unnormalised partial
// (m, l, o[D]) per query head: m is the max logit in log2 units
// (logit * log2 e), l = sum 2^(s - m), o = sum 2^(s - m) * v. The merge
// kernel combines the nsplit + 1 partials of each (sequence, kv head) in
// index order, so results do not depend on scheduling.
//
// INT4 chunk, per wave (a quarter of the chunk):
//  * The kept positions (keep-mask bits) are compacted into an LDS list of
//    token-record indices, so evicted tokens cost no HBM reads: each lane
//    loads one mask word and the block-table entries of its two pages, and a
//    ballot scan of the lanes' popcounts gives each lane where its records go.
//  * The list is walked in 32-token tiles, each as two steps: a K step (K
//    codes and K meta) that writes the tile's logits to LDS, raises the
//    running max per head and rescales the accumulators once, and a V step
//    (V codes and V meta, whose line the K step has just brought into L2)
//    that accumulates P.V with p = 2^(s - max). The steps form one stream
//    behind a ring of kRing register tiles, so the loads of the next steps
//    are in flight during each step's arithmetic.
//  * Logits use v_mfma_f32_16x16x32_f16 with the raw codes: a nibble n becomes
//    the fp16 value 1024 + n (or 1024 + 16n) by OR-ing it into 0x6400, which is
//    exact; one MFMA row is one token, one column one (group, head) pair, and
//    the query operand (q, zero outside the column's own group) makes
//    each column accumulate exactly one group's dot product. The accumulators
//    start at -sum(q) * 1024, so the offset cancels inside the MFMA; the
//    per-group scale and min are then applied in float32:
//      s = sum_g scale_g (q_g . c_g) + min_g sum(q_g)   (rows = tokens).
//    The exponentials 2^(s - max) are taken once per (token, head) and left
//    in LDS for the V step.
//  * P.V uses the same MFMA with rows = (group, head) pairs, whose P operand
//    is p * V_scale[token][group] in fp16, and columns = channels 8n + m read
//    from V-code dword n; the codes enter as the exact fp16 subnormals
//    c * 2^-24 or c * 2^-20 (one AND each, no offset). One more MFMA against
//    a constant 1.0 operand sums the fp16 P operand per row, which centres the
//    codes at 8: the fp16 rounding of P then weighs (c - 8) instead of c. Only
//    rows whose group matches the column's channel group are kept. The side
//    term sum_t p_t V_min + 8 p_t V_scale is accumulated in float32.
#include "kvc_internal.h"

#include <type_traits>

namespace kvc {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr uint32_t kMagic = 0x64006400u;   // fp16 1024.0 in both halves
constexpr uint32_t kOne = 0x3C003C00u;     // fp16 1.0 in both halves
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kRing = 4;  // INT4 steps in flight per wave (the one in use plus three prefetched)
static_assert(kRing % 2 == 0, "ring slots alternate between K and V steps");
static_assert(kMaxChunk / kWaves <= 64 * 32, "the compaction gives each lane one mask word of a wave's range");

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef float float2v __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

struct AttnParams {
  const void* q;
  const uint8_t* codes;
  const uint16_t* meta;
  const int8_t* codes8;
  const float* scales8;
  const int32_t* block_table;
  const int32_t* seq_lens;
  const uint32_t* mask;
  float* parts;  // [B][Hkv][nsplit + 1][G][2 + D]
  float* out;
  float* lse;
  float alpha;  // softmax scale * log2(e)
  int batch;
  int int8_first;  // dispatch the INT8-region workgroups before the INT4 chunks
  int hkv;
  int max_pages;
  int num_pages;
  int max_ctx;
  int words;
  int chunk;
  int nsplit;
  int window;  // > 0: only the last `window` INT4-region positions are read
  int sink, recent;  // INT8-protected sink and recent positions (16/128, or 0/0)
  const uint8_t* codes_h;  // host tier: pages [num_pages, num_pages + host_pages)
  const uint16_t* meta_h;
  int host_pages;
};

__device__ inline float h2f(uint32_t bits16) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}

__device__ inline half8 as_half8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  const u32x4 v = {a, b, c, d};
  return __builtin_bit_cast(half8, v);
}

__device__ inline uint32_t pack_f16x2(float a, float b) {
  const float2v v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, half2v));
}

__device__ inline float4v mfma16x16x32(half8 a, half8 b, float4v c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// (x & m) | c in one VALU op: gfx950's three-input bitwise op with truth
// table 0xEA (bit i of the table is f(a, b, c) for i = 4a + 2b + c).
// Written out because the compiler emits a separate and + or otherwise.
__device__ inline uint32_t and_or(uint32_t x, uint32_t m, uint32_t c) {
  return __builtin_amdgcn_bitop3_b32(x, m, c, 0xEA);
}

// Rotate right by N lanes within each row of 16 lanes.
template <int N>
__device__ inline float row_ror(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x120 + N, 0xF, 0xF, true));
}

// Reductions over the four rows of 16 lanes (lanes n, n+16, n+32, n+48) with
// the gfx950 lane-swap instructions. The swap returns both registers as a
// pair; it is read through a 64-bit view because indexing the returned
// vector element-wise selects the first register twice in this compiler.
__device__ inline void swap32(float v, float& a, float& b) {
  const uint32_t u = __builtin_bit_cast(uint32_t, v);
  const uint64_t w = __builtin_bit_cast(uint64_t, __builtin_amdgcn_permlane32_swap(u, u, false, false));
  a = __builtin_bit_cast(float, (uint32_t)w);
  b = __builtin_bit_cast(float, (uint32_t)(w >> 32));
}
__device__ inline void swap16(float v, float& a, float& b) {
  const uint32_t u = __builtin_bit_cast(uint32_t, v);
  const uint64_t w = __builtin_bit_cast(uint64_t, __builtin_amdgcn_permlane16_swap(u, u, false, false));
  a = __builtin_bit_cast(float, (uint32_t)w);
  b = __builtin_bit_cast(float, (uint32_t)(w >> 32));
}
__device__ inline float rows_max(float v) {
  float a, b;
  swap32(v, a, b);
  swap16(fmaxf(a, b), a, b);
  return fmaxf(a, b);
}
__device__ inline float rows_sum(float v) {
  float a, b;
  swap32(v, a, b);
  swap16(a + b, a, b);
  return a + b;
}

// Reductions over all 64 lanes: DPP rotations within each row, then the rows.
__device__ inline float wave_max(float v) {
  v = fmaxf(v, row_ror<1>(v));
  v = fmaxf(v, row_ror<2>(v));
  v = fmaxf(v, row_ror<4>(v));
  v = fmaxf(v, row_ror<8>(v));
  return rows_max(v);
}
__device__ inline float wave_sum(float v) {
  v += row_ror<1>(v);
  v += row_ror<2>(v);
  v += row_ror<4>(v);
  v += row_ror<8>(v);
  return rows_sum(v);
}

template <bool QBF16>
__device__ inline float load_q(const void* q, size_t off) {
  if constexpr (QBF16) return __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(q)[off] << 16);
  else return reinterpret_cast<const float*>(q)[off];
}

template <int D, int G>
struct Shape {
  static constexpr int NG = D / 32;   // quantisation groups per row = QK MFMAs per 16 tokens
  static constexpr int SB = D / 8;    // K-code bytes held per lane slot
  static constexpr int VD = D / 8;    // V-code dwords per token
  static constexpr int NC = NG * G;   // distinct (group, head) columns, <= 16
};

// LDS of one workgroup. The INT4 path gives each wave its own region (kept
// list, pass-1 logits - later reused for the wave's output -, and staging for
// one tile of V codes and meta); the INT8 path overlays its own buffers.
template <int D, int G>
struct Smem {
  static constexpr int kListCap = kMaxChunk / kWaves;  // positions per wave
  // Row strides padded so that the 16-lane row groups of a wave fall into
  // different LDS banks on the P.V operand reads.
  static constexpr int kLgStride = 48;    // 32 logits + 16
  static constexpr int kVStride = D / 8 + 4;
  struct Wave4 {
    union {
      uint32_t rec[kListCap + 32];        // token-record indices, padded with copies
      float o[G][D];                      // the wave's unnormalised output (after the list)
    } ro;
    float logit[G][kLgStride];            // the current tile's logits / alpha, then p
    uint32_t vbuf[32][kVStride];          // V codes of the current 32 tokens
    uint32_t mbuf[32][D / 32];            // K or V (scale | min << 16) of the current 32 tokens
  };
  struct Int8 {
    float q[G][D];
    int8_t vcode[kWaves][36][D];
    float p[kWaves][36][G];
    float o[kWaves][G][D];
  };
  union {
    Wave4 w4[kWaves];
    Int8 i8;
  } u;
  float m[kWaves][G];
  float l[kWaves][G];
  float vm[kWaves][16];
};

// Combine the four waves' (m, l, o) held in LDS into one partial and store it.
template <int D, int G, typename OF>
__device__ inline void store_partial(Smem<D, G>& sm, OF o_of, float* dst) {
  const int tid = threadIdx.x;
  for (int i = tid; i < G * D; i += kThreads) {
    const int h = i / D, ch = i % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sm.m[w][h]);
    float o = 0.0f, l = 0.0f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float mw = sm.m[w][h];
        if (mw == -INFINITY) continue;
        const float a = __builtin_amdgcn_exp2f(mw - M);
        o += a * o_of(w)[h * D + ch];
        l += a * sm.l[w][h];
      }
    }
    float* row = dst + (size_t)h * (2 + D);
    row[2 + ch] = o;
    if (ch == 0) { row[0] = M; row[1] = l; }
  }
}

// ------------------------------------------------------------------ INT4 chunk
// Per wave: compact the kept positions of its quarter of the chunk, then walk
// them in 32-token tiles, each a K step (logits, running max, one rescale)
// followed by a V step (P.V), with the next steps' loads in flight.
template <int D, int G, bool QBF16, bool TIER>
__device__ void int4_chunk(const AttnParams& p, Smem<D, G>& sm, int b, int kvh, int split) {
  using S = Shape<D, G>;
  constexpr int NG = S::NG, VD = S::VD, NC = S::NC;
  constexpr int MH = NG / 2;  // meta words per half row (K or V part)
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int s = lane >> 4;         // row slot
  const int n = lane & 15;         // column
  const int gc = (n / G) % NG;     // column's group
  const int hc = n % G;            // column's head
  const int tl = lane >> 1;        // token this lane stages (compact loads)
  const int hf = lane & 1;         // which half of that token's row
  auto& wv = sm.u.w4[wave];
  int L = p.seq_lens[b];
  L = L < 0 ? 0 : (L > p.max_ctx ? p.max_ctx : L);
  const int slots = p.sink + p.recent;
  const int n4 = L > slots ? L - slots : 0;
  // INT4 region [r0, r1), or its last `window` positions; chunks start at
  // base (0, or the window's start rounded down to 64 positions)
  int r0 = p.sink, base = 0;
  const int r1 = p.sink + n4;
  if (p.window > 0 && r1 - p.window > r0) {
    r0 = r1 - p.window;
    base = r0 & ~63;
  }
  const int q4 = p.chunk / kWaves;
  const int w0 = base + split * p.chunk + wave * q4;
  const int lo = w0 > r0 ? w0 : r0;
  const int hi = w0 + q4 < r1 ? w0 + q4 : r1;

  // The query entries this lane feeds to the QK product (code s*D/4 + 8m + perm[r]
  // of its column's head), loaded first so their latency overlaps the compaction.
  float qraw[NG][8];
  {
    // the lane's D/4 query entries are contiguous: a few 16-byte loads
    constexpr int NE = D / 4;
    const size_t qoff = ((size_t)b * p.hkv * G + kvh * G + hc) * D + s * NE;
    float qe[NE];
    if constexpr (QBF16) {
      const u32x4* qp = reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(p.q) + qoff);
#pragma unroll
      for (int i = 0; i < NE / 8; ++i) {
        const u32x4 x = qp[i];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          qe[8 * i + 2 * k] = __uint_as_float(x[k] << 16);
          qe[8 * i + 2 * k + 1] = __uint_as_float(x[k] & 0xFFFF0000u);
        }
      }
    } else {
      const float4v* qp = reinterpret_cast<const float4v*>(reinterpret_cast<const float*>(p.q) + qoff);
#pragma unroll
      for (int i = 0; i < NE / 4; ++i) {
        const float4v x = qp[i];
#pragma unroll
        for (int k = 0; k < 4; ++k) qe[4 * i + k] = x[k];
      }
    }
    const int perm[8] = {0, 4, 1, 5, 2, 6, 3, 7};
#pragma unroll
    for (int m = 0; m < NG; ++m)
#pragma unroll
      for (int r = 0; r < 8; ++r) qraw[m][r] = qe[8 * m + perm[r]];
  }

  // ---- compact the kept positions of this wave's range into an LDS list.
  // Lane l owns mask word l of the range (positions w0 + 32l .. + 31, at most
  // 64 words) and the block-table entries of its two pages; a bit-sliced
  // ballot scan gives each lane its offset, and each lane writes its kept
  // records in position order, so the list is in position order.
  uint32_t* list = wv.ro.rec;
  int cnt = 0;
  {
    const uint32_t* mrow = p.mask + ((size_t)b * p.hkv + kvh) * p.words;
    const int32_t* bt = p.block_table + (size_t)b * p.max_pages;
    const int p0 = w0 + 32 * lane;  // first position of the lane's word
    uint32_t word = 0;
    int32_t pga = -1, pgb = -1;
    if (lane < q4 / 32 && p0 < hi) {
      word = mrow[p0 >> 5];
      pga = bt[p0 >> 4];
      if (p0 + 16 < hi) pgb = bt[(p0 >> 4) + 1];
    }
    // keep positions in [lo, hi) of valid pages only
    const int from = lo - p0, to = hi - p0;  // bit range [from, to) of the word
    if (to <= 0 || from >= 32) word = 0;
    else {
      if (from > 0) word &= ~0u << from;
      if (to < 32) word &= (1u << to) - 1u;
    }
    const int lim = p.num_pages + p.host_pages;
    if (pga < 0 || pga >= lim) word &= 0xFFFF0000u;
    if (pgb < 0 || pgb >= lim) word &= 0x0000FFFFu;
    // exclusive prefix of the lanes' popcounts (each <= 32: six bit planes)
    const uint32_t pc = (uint32_t)__popc(word);
    int off = 0;
#pragma unroll
    for (int bit = 0; bit < 6; ++bit) {
      const uint64_t plane = __ballot((pc >> bit) & 1u);
      const int below = __builtin_amdgcn_mbcnt_hi((uint32_t)(plane >> 32),
                                                  __builtin_amdgcn_mbcnt_lo((uint32_t)plane, 0));
      off += below << bit;
      cnt += __popcll(plane) << bit;
    }
    const uint32_t rec_a = ((uint32_t)pga * p.hkv + kvh) * kPage;
    const uint32_t rec_b = ((uint32_t)pgb * p.hkv + kvh) * kPage;
    while (word != 0) {
      const int bit = __builtin_ctz(word);
      word &= word - 1u;
      list[off++] = (bit < 16 ? rec_a : rec_b) + (uint32_t)(bit & 15);
    }
  }
  cnt = __builtin_amdgcn_readfirstlane(cnt);  // wave-uniform: keeps the main loop scalar
  // Pad the list with copies of its first entry to a whole number of ring
  // turns (kRing steps = kRing / 2 tiles), so the unrolled main loop needs no
  // per-step guard: a guard there turns into divergent branches, across which
  // the compiler can only drain every outstanding load. Padded tokens get p = 0.
  constexpr int kTurn = 16 * kRing;  // tokens per ring turn
  const int padded = (cnt + kTurn - 1) / kTurn * kTurn;
  if (cnt > 0) {
    const uint32_t fill = list[0];
    for (int i = cnt + lane; i < padded; i += 64) list[i] = fill;
  }

  // Per lane: m_col and l_col belong to head hc (the lane's column head),
  // vm1/vm2 to accumulator row (gc, hc) of the P operand; acc holds P.V with
  // rows (group, head) and columns channels, acc_one = sum of the fp16 P
  // operand per row.
  float m_col = -INFINITY, l_col = 0.0f, vm1 = 0.0f, vm2 = 0.0f;
  float4v acc[8], acc_one = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int m = 0; m < 8; ++m) acc[m] = acc_one;

  if (cnt > 0) {
    // ---- query operands: column (gc, hc) holds q for group gc only, divided
    // by 16 in the k slots whose codes enter as 1024 + 16c (exact in fp16 for
    // a bf16 query)
    const int slot_group = (s * D / 4) / 32;
    const bool active = slot_group == gc;
    const float alpha = p.alpha;
    half8 bq[NG];
    float off = 0.0f, qs = 0.0f;
#pragma unroll
    for (int m = 0; m < NG; ++m) {
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const bool x16 = (r == 2 || r == 3 || r == 6 || r == 7);
        const float qv = active ? qraw[m][r] : 0.0f;
        qs += qv;
        const _Float16 qh = (_Float16)(x16 ? qv * 0.0625f : qv);
        bq[m][r] = qh;
        off += (float)qh * 1024.0f;
      }
    }
    // every code of the column's group sits in exactly one active slot
    off = rows_sum(off);
    qs = rows_sum(qs);
    // QK accumulators start at -off, which removes the 1024 of every code
    const float4v offv = {-off, -off, -off, -off};
    const uint8_t* kbase = p.codes + s * S::SB;
    // V pieces: 4 lanes per token at D = 128, 2 at D = 64, 16 bytes each
    const uint8_t* vbase = p.codes + D / 2 + (D == 128 ? 16 * (lane & 3) : 16 * (lane & 1));
    const uint8_t* mbase = reinterpret_cast<const uint8_t*>(p.meta) + hf * (MH * 4);
    // Host tier: records from rec_h0 on belong to host pages; the same
    // record arithmetic applies from bases shifted back by rec_h0 records.
    const uint32_t rec_h0 = (uint32_t)p.num_pages * p.hkv * kPage;
    const uint8_t* kbase_h = nullptr;
    const uint8_t* vbase_h = nullptr;
    const uint8_t* mbase_h = nullptr;
    if constexpr (TIER) {
      const uintptr_t ch = reinterpret_cast<uintptr_t>(p.codes_h) - (uintptr_t)rec_h0 * D;
      const uintptr_t mh = reinterpret_cast<uintptr_t>(p.meta_h) - (uintptr_t)rec_h0 * (D / 4);
      kbase_h = reinterpret_cast<const uint8_t*>(ch) + (kbase - p.codes);
      vbase_h = reinterpret_cast<const uint8_t*>(ch) + (vbase - p.codes);
      mbase_h = reinterpret_cast<const uint8_t*>(mh) + hf * (MH * 4);
    }
    // address of record `rec` from a device-pool base and its host-tier twin
    auto at = [&](const uint8_t* dev, const uint8_t* hst, uint32_t rec, uint32_t stride) {
      if constexpr (TIER) return (rec >= rec_h0 ? hst : dev) + (uint64_t)rec * stride;
      else return dev + (uint64_t)rec * stride;
    };
    const int ntile = padded >> 5;  // 32-token tiles
    const int nstep = 2 * ntile;    // K step, then V step, per tile; a multiple of kRing

    // One stream of steps: step 2j brings K codes and K meta of tile j, step
    // 2j + 1 the V codes and V meta of the same tokens. The V half of a token
    // record shares the 128-byte line of its K half, so it is read from L2
    // right after the K step brought the line in. Both kinds load the same
    // registers with the same instructions (two loads of NG code dwords, one
    // of MH meta dwords), so the ring never drains between them.
    struct Tile {
      uint32_t c[2 * NG];
      uint32_t mh[MH];
    };
    // kind: true for a K step, false for a V step; steps past the end reload
    // the last tile (L2 hits, results unused)
    auto fetch = [&](auto kind, int step, Tile& t) {
      constexpr bool isk = decltype(kind)::value;
      const int tile = step >> 1;
      const int it = 32 * (tile < ntile ? tile : ntile - 1);
      const uint32_t rt = list[it + tl];
      const uint8_t* a0;
      const uint8_t* a1;
      if constexpr (isk) {
        // lane (s, n): K slot s of tokens n and 16 + n (4 lanes per token row)
        a0 = at(kbase, kbase_h, list[it + n], D);
        a1 = at(kbase, kbase_h, list[it + 16 + n], D);
      } else if constexpr (D == 128) {
        // lane (t, j): 16-byte piece j of the V codes of tokens t and 16 + t
        a0 = at(vbase, vbase_h, list[it + (lane >> 2)], D);
        a1 = at(vbase, vbase_h, list[it + 16 + (lane >> 2)], D);
      } else {
        // lane (t, j): 16-byte piece j of the V codes of token t
        a0 = at(vbase, vbase_h, list[it + (lane >> 1)], D);
        a1 = a0;
      }
      const uint8_t* am = at(mbase, mbase_h, rt, D / 4) + (isk ? 0 : D / 8);
      if constexpr (D == 128) {
        const u32x4 x = *reinterpret_cast<const u32x4*>(a0);
        const u32x4 y = *reinterpret_cast<const u32x4*>(a1);
        const u32x2 mm = *reinterpret_cast<const u32x2*>(am);
#pragma unroll
        for (int m = 0; m < 4; ++m) { t.c[m] = x[m]; t.c[4 + m] = y[m]; }
        t.mh[0] = mm[0];
        t.mh[1] = mm[1];
      } else if constexpr (isk) {
        const u32x2 x = *reinterpret_cast<const u32x2*>(a0);
        const u32x2 y = *reinterpret_cast<const u32x2*>(a1);
#pragma unroll
        for (int m = 0; m < 2; ++m) { t.c[m] = x[m]; t.c[2 + m] = y[m]; }
        t.mh[0] = *reinterpret_cast<const uint32_t*>(am);
      } else {
        const u32x4 x = *reinterpret_cast<const u32x4*>(a0);
#pragma unroll
        for (int m = 0; m < 4; ++m) t.c[m] = x[m];
        t.mh[0] = *reinterpret_cast<const uint32_t*>(am);
      }
    };

    // ---- K step: logits of 32 tokens, running max, rescale when it rises,
    // then p = 2^(s - max) of every (token, head) once, into LDS
    auto compute1 = [&](const Tile& t, int it) {
#pragma unroll
      for (int m = 0; m < MH; ++m) wv.mbuf[tl][hf * MH + m] = t.mh[m];
      __builtin_amdgcn_wave_barrier();
      // QK: C[token][(g,h)] = q_g . c_g (codes taken as 1024 + c)
      float4v c0 = offv, c1 = offv;
#pragma unroll
      for (int m = 0; m < NG; ++m) {
        uint32_t x = t.c[m];
        uint32_t y = x >> 8;
        half8 a = as_half8(and_or(x, 0x000F000Fu, kMagic), and_or(x, 0x00F000F0u, kMagic),
                           and_or(y, 0x000F000Fu, kMagic), and_or(y, 0x00F000F0u, kMagic));
        c0 = mfma16x16x32(a, bq[m], c0);
        x = t.c[NG + m];
        y = x >> 8;
        a = as_half8(and_or(x, 0x000F000Fu, kMagic), and_or(x, 0x00F000F0u, kMagic),
                     and_or(y, 0x000F000Fu, kMagic), and_or(y, 0x00F000F0u, kMagic));
        c1 = mfma16x16x32(a, bq[m], c1);
      }
      // u_g = scale_g (q_g . c_g) + min_g sum(q_g); the logit in log2 units is
      // alpha * sum_g u_g, with alpha applied in the exponent below
      float sv[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int tok = i < 4 ? 4 * s + i : 16 + 4 * s + (i - 4);
        const uint32_t km = wv.mbuf[tok][gc];
        const float d = i < 4 ? c0[i] : c1[i - 4];
        sv[i] = fmaf(h2f(km & 0xFFFFu), d, fmaf(h2f(km >> 16), qs, 0.0f));
      }
      // sum the group columns of each head (columns h, h+G, h+2G, ... within a row)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if constexpr (NC >= 2 * G) sv[i] += row_ror<G>(sv[i]);
        if constexpr (NC >= 4 * G) sv[i] += row_ror<2 * G>(sv[i]);
        if constexpr (NC >= 8 * G) sv[i] += row_ror<4 * G>(sv[i]);
        if constexpr (NC >= 16 * G) sv[i] += row_ror<8 * G>(sv[i]);
      }
      // Padding tokens past cnt repeat list[0], whose logit tile 0 has already
      // folded into the max, so they cannot raise it; they get p = 0 below.
      float tmax = sv[0];
#pragma unroll
      for (int i = 1; i < 8; ++i) tmax = fmaxf(tmax, sv[i]);
      if (n < G) {
        const float4v lo4 = {sv[0], sv[1], sv[2], sv[3]};
        const float4v hi4 = {sv[4], sv[5], sv[6], sv[7]};
        *reinterpret_cast<float4v*>(&wv.logit[n][4 * s]) = lo4;
        *reinterpret_cast<float4v*>(&wv.logit[n][16 + 4 * s]) = hi4;
      }
      // every tile holds at least one kept token, so the new max is finite
      // (m_col is in log2 units, alpha > 0)
      const float mnew = fmaxf(m_col, alpha * rows_max(tmax));
      if (__ballot(mnew > m_col) != 0) {
        const float f = __builtin_amdgcn_exp2f(m_col - mnew);  // 0 on the first tile
        l_col *= f;
        vm1 *= f;
        vm2 *= f;
        // accumulator row 4s + j belongs to head j % G (G divides 4); lane
        // h < G has column (0, h), so it holds head h's factor
        float fh[G];
#pragma unroll
        for (int h = 0; h < G; ++h)
          fh[h] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, f), h));
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float fj = fh[j % G];
#pragma unroll
          for (int m = 0; m < 8; ++m) acc[m][j] *= fj;
          acc_one[j] *= fj;
        }
      }
      m_col = mnew;
      __builtin_amdgcn_wave_barrier();
      // p for (head hc, tokens of this lane): 2 per lane at G = 4, 1 at G = 2,
      // 1 on half the lanes at G = 1
      const int lim = cnt - it;  // tokens of this tile below lim are real
      if constexpr (G == 4) {
        const int k2 = 2 * (4 * s + n / 4);
        float2v lg = *reinterpret_cast<const float2v*>(&wv.logit[hc][k2]);
        lg[0] = k2 < lim ? __builtin_amdgcn_exp2f(fmaf(alpha, lg[0], -m_col)) : 0.0f;
        lg[1] = k2 + 1 < lim ? __builtin_amdgcn_exp2f(fmaf(alpha, lg[1], -m_col)) : 0.0f;
        l_col += lg[0] + lg[1];
        *reinterpret_cast<float2v*>(&wv.logit[hc][k2]) = lg;
      } else {
        const int k = G == 2 ? 8 * s + n / 2 : 16 * s + n;
        if (k < 32) {
          const float pr = k < lim ? __builtin_amdgcn_exp2f(fmaf(alpha, wv.logit[hc][k], -m_col)) : 0.0f;
          l_col += pr;
          wv.logit[hc][k] = pr;
        }
      }
      __builtin_amdgcn_wave_barrier();
    };

    // ---- V step: P.V of the same 32 tokens. V codes enter the MFMA as the
    // exact fp16 subnormals c * 2^-24 (low nibble of a half) and c * 2^-20
    // (second nibble), so no offset has to be removed afterwards.
    const int vdw = n % VD;
    auto compute2 = [&](const Tile& t) {
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        if constexpr (D == 128) {
          wv.vbuf[lane >> 2][4 * (lane & 3) + m] = t.c[m];
          wv.vbuf[16 + (lane >> 2)][4 * (lane & 3) + m] = t.c[4 + m];
        } else {
          wv.vbuf[lane >> 1][4 * (lane & 1) + m] = t.c[m];
        }
      }
#pragma unroll
      for (int m = 0; m < MH; ++m) wv.mbuf[tl][hf * MH + m] = t.mh[m];
      __builtin_amdgcn_wave_barrier();
      const float4v pv0 = *reinterpret_cast<const float4v*>(&wv.logit[hc][4 * s]);
      const float4v pv1 = *reinterpret_cast<const float4v*>(&wv.logit[hc][16 + 4 * s]);
      uint32_t vd[8];
      float pp[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int tok = i < 4 ? 4 * s + i : 16 + 4 * s + (i - 4);
        vd[i] = wv.vbuf[tok][vdw];
        const uint32_t vmeta = wv.mbuf[tok][gc];
        const float pr = i < 4 ? pv0[i] : pv1[i - 4];
        const float ps = fmaf(pr, h2f(vmeta & 0xFFFFu), 0.0f);
        vm1 = fmaf(pr, h2f(vmeta >> 16), vm1);
        vm2 += ps;
        pp[i] = ps;
      }
      const half8 A = as_half8(pack_f16x2(pp[0], pp[1]), pack_f16x2(pp[2], pp[3]),
                               pack_f16x2(pp[4], pp[5]), pack_f16x2(pp[6], pp[7]));
      // V codes of tokens (2q, 2q+1) paired into the halves of one dword
      uint32_t xv[8];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        xv[q] = __builtin_amdgcn_perm(vd[2 * q + 1], vd[2 * q], 0x05040100u);      // channels 0..3
        xv[4 + q] = __builtin_amdgcn_perm(vd[2 * q + 1], vd[2 * q], 0x07060302u);  // channels 4..7
      }
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        uint32_t bw[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t x = xv[(m / 4) * 4 + q];
          const uint32_t y = (m & 2) ? x >> 8 : x;
          bw[q] = y & ((m & 1) ? 0x00F000F0u : 0x000F000Fu);
        }
        acc[m] = mfma16x16x32(A, as_half8(bw[0], bw[1], bw[2], bw[3]), acc[m]);
      }
      acc_one = mfma16x16x32(A, as_half8(kOne, kOne, kOne, kOne), acc_one);
      __builtin_amdgcn_wave_barrier();
    };

    // slot j of the ring always holds a step of parity j, so every unrolled
    // slot knows its kind at compile time
    using KStep = std::integral_constant<bool, true>;
    using VStep = std::integral_constant<bool, false>;
    Tile ring[kRing];
#pragma unroll
    for (int j = 0; j < kRing - 1; ++j) {
      if (j % 2 == 0) fetch(KStep{}, j, ring[j]);
      else fetch(VStep{}, j, ring[j]);
    }
    for (int step = 0; step < nstep; step += kRing) {
#pragma unroll
      for (int j = 0; j < kRing; ++j) {
        if ((j + kRing - 1) % 2 == 0) fetch(KStep{}, step + j + kRing - 1, ring[(j + kRing - 1) % kRing]);
        else fetch(VStep{}, step + j + kRing - 1, ring[(j + kRing - 1) % kRing]);
        if (j % 2 == 0) compute1(ring[j], 16 * (step + j));
        else compute2(ring[j]);
      }
    }
    // l: sum over the lanes of each head (all rows, columns h, h+G, ...)
    l_col = rows_sum(l_col);
    if constexpr (G < 16) l_col += row_ror<G>(l_col);
    if constexpr (2 * G < 16) l_col += row_ror<2 * G>(l_col);
    if constexpr (4 * G < 16) l_col += row_ror<4 * G>(l_col);
    if constexpr (8 * G < 16) l_col += row_ror<8 * G>(l_col);
    vm1 = rows_sum(vm1);
    vm2 = rows_sum(vm2);
  }

  // ---- this wave's (m, l, o) into LDS (o reuses the list area)
  if (lane < G) {
    sm.m[wave][lane] = m_col;  // lane h < G has column (0, h)
    sm.l[wave][lane] = l_col;
  }
  // side term of row (g, h): sum_t p (V_min + 8 V_scale)
  if (lane < 16) sm.vm[wave][lane] = fmaf(8.0f, vm2, vm1);
  __builtin_amdgcn_s_waitcnt(0);
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int row = 4 * s + j;
    const int g = (row / G) % NG, h = row % G;
    const bool ok = row < NC && g == n / 4 && n < VD && cnt > 0;
    if (ok) {
      // channel 8n + m: sum p V_scale c, with c entering as c * 2^-24 (m even)
      // or c * 2^-20 (m odd); minus 8 sum p V_scale re-centres the codes
      const float side = sm.vm[wave][g * G + h] - 8.0f * acc_one[j];
#pragma unroll
      for (int m = 0; m < 8; ++m)
        wv.ro.o[h][8 * n + m] = fmaf(acc[m][j], (m & 1) ? 1048576.0f : 16777216.0f, side);
    }
  }
  if (cnt == 0) {
    for (int i = lane; i < G * D; i += 64) wv.ro.o[i / D][i % D] = 0.0f;
  }
}

// ------------------------------------------------------------------ INT8 region
// The <= 144 protected positions of one (sequence, kv head) in float32: each
// wave takes 36 slots, lane = slot for the logits, lane = channels for P.V.
// Which slots hold attended positions follows from L alone: all 144 when
// L >= 144, else exactly slots [0, L) (slot = position below 144). So every
// slot's codes and scales are loaded at once, together with the query and the
// length, and masked afterwards; the region's sums do not depend on order.
template <int D, int G, bool QBF16>
__device__ void int8_region(const AttnParams& p, Smem<D, G>& sm, int b, int kvh) {
  constexpr int CPL = D / 64;
  constexpr int NW = D / 16;  // 16-byte words per K (or V) row
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int slot = wave * 36 + lane;
  const int slots = p.sink + p.recent;  // 144, or 0 without INT8 protection
  const bool inr = lane < 36 && slot < slots;
  const size_t base = ((size_t)b * p.hkv + kvh) * slots;
  u32x4 kw[NW];
  float2v sc = {0.0f, 0.0f};
  if (inr) {
    const u32x4* row = reinterpret_cast<const u32x4*>(p.codes8 + (base + slot) * 2 * D);
#pragma unroll
    for (int i = 0; i < NW; ++i) kw[i] = row[i];
    u32x4 vw[NW];
#pragma unroll
    for (int i = 0; i < NW; ++i) vw[i] = row[NW + i];
    sc = *reinterpret_cast<const float2v*>(p.scales8 + (base + slot) * 2);
#pragma unroll
    for (int i = 0; i < NW; ++i) *reinterpret_cast<u32x4*>(&sm.u.i8.vcode[wave][lane][16 * i]) = vw[i];
  }
  for (int i = threadIdx.x; i < G * D; i += kThreads) {
    const int h = i / D, d = i % D;
    sm.u.i8.q[h][d] = load_q<QBF16>(p.q, ((size_t)b * p.hkv * G + kvh * G + h) * D + d) * p.alpha;
  }
  int L = p.seq_lens[b];
  L = L < 0 ? 0 : (L > p.max_ctx ? p.max_ctx : L);
  const int nvalid = L < slots ? L : slots;
  const int cntw = nvalid - wave * 36 < 0 ? 0 : (nvalid - wave * 36 > 36 ? 36 : nvalid - wave * 36);
  const bool valid = lane < cntw;
  __syncthreads();
  float s[G];
#pragma unroll
  for (int h = 0; h < G; ++h) s[h] = -INFINITY;
  if (valid) {
    float dot[G];
#pragma unroll
    for (int h = 0; h < G; ++h) dot[h] = 0.0f;
#pragma unroll
    for (int i = 0; i < NW; ++i) {
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const float c = (float)(int8_t)(kw[i][k / 4] >> (8 * (k % 4)));
#pragma unroll
        for (int h = 0; h < G; ++h) dot[h] = fmaf(sm.u.i8.q[h][16 * i + k], c, dot[h]);
      }
    }
#pragma unroll
    for (int h = 0; h < G; ++h) s[h] = sc[0] * dot[h];
  }
  // p of slot j for the G heads, side by side, so the P.V loop reads them at once
  float m[G], l[G], o[G][CPL];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float mx = wave_max(s[h]);
    m[h] = mx;
    const float pr = valid ? __builtin_amdgcn_exp2f(s[h] - mx) : 0.0f;
    l[h] = wave_sum(pr);
    if (lane < 36) sm.u.i8.p[wave][lane][h] = pr * sc[1];
#pragma unroll
    for (int c = 0; c < CPL; ++c) o[h][c] = 0.0f;
  }
  __builtin_amdgcn_s_waitcnt(0);
  __builtin_amdgcn_wave_barrier();
  // P.V over all 36 slots of the wave: slots past cntw have p = 0 (their
  // codes are whatever the buffer holds, always finite), so the loop has a
  // fixed trip count and its LDS reads can be issued together
#pragma unroll 12
  for (int j = 0; j < 36; ++j) {
    float pj[G];
#pragma unroll
    for (int h = 0; h < G; ++h) pj[h] = sm.u.i8.p[wave][j][h];
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const float v = (float)sm.u.i8.vcode[wave][j][lane * CPL + c];
#pragma unroll
      for (int h = 0; h < G; ++h) o[h][c] = fmaf(pj[h], v, o[h][c]);
    }
  }
  if (lane < G) {
#pragma unroll
    for (int h = 0; h < G; ++h)
      if (lane == h) { sm.m[wave][h] = cntw > 0 ? m[h] : -INFINITY; sm.l[wave][h] = cntw > 0 ? l[h] : 0.0f; }
  }
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int c = 0; c < CPL; ++c) sm.u.i8.o[wave][h][lane * CPL + c] = o[h][c];
}

// ------------------------------------------------------------------ merge
// One wave per (query head, kv head, sequence) merges the partials in a fixed
// order (outputs summed in index order): M = max_j m_j, w_j = 2^(m_j - M) (0 for empty partials),
// out = sum_j w_j o_j / sum_j w_j l_j, lse = ln 2 * (M + log2 sum_j w_j l_j).
// Lane l owns output channels [l*CPL, l*CPL + CPL); the (m, l) pairs and the
// lane's slices of the first kPre partials are loaded together up front.
template <int D, int G>
__global__ __launch_bounds__(64) void merge_kernel(AttnParams p) {
  constexpr int CPL = D / 64;  // channels per lane
  constexpr int kPre = 32;     // partials whose slices are loaded up front
  typedef float fcpl __attribute__((ext_vector_type(CPL)));
  __shared__ float wts[kMaxParts];
  const int h = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x;
  const int np = p.nsplit + 1;
  const float* parts = p.parts + ((size_t)b * p.hkv + kvh) * np * G * (2 + D) + (size_t)h * (2 + D);
  const size_t pstride = (size_t)G * (2 + D);
  fcpl pre[kPre];
#pragma unroll
  for (int j = 0; j < kPre; ++j) {
    const int jj = j < np ? j : np - 1;
    pre[j] = *reinterpret_cast<const fcpl*>(parts + jj * pstride + 2 + CPL * lane);
  }
  // (m, l) of partials lane, lane + 64, ...: at most kMaxParts / 64 per lane
  constexpr int kML = kMaxParts / 64;
  float mj[kML], lj[kML];
#pragma unroll
  for (int r = 0; r < kML; ++r) {
    const int j = lane + 64 * r;
    mj[r] = -INFINITY;
    lj[r] = 0.0f;
    if (j < np) {
      const float2v ml = *reinterpret_cast<const float2v*>(parts + j * pstride);
      mj[r] = ml[0];
      lj[r] = ml[1];
    }
  }
  float M = -INFINITY;
#pragma unroll
  for (int r = 0; r < kML; ++r) M = fmaxf(M, mj[r]);
  M = wave_max(M);
  float den = 0.0f;
#pragma unroll
  for (int r = 0; r < kML; ++r) {
    const int j = lane + 64 * r;
    const float w = (mj[r] == -INFINITY || M == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(mj[r] - M);
    den += w * lj[r];
    if (j < np) wts[j] = w;
  }
  den = wave_sum(den);
  __builtin_amdgcn_wave_barrier();  // one wave: its LDS writes are seen by its later reads
  fcpl acc = {};
#pragma unroll
  for (int j = 0; j < kPre; ++j)
    if (j < np) acc += wts[j] * pre[j];
  // every partial is written by the attention kernel, so no load is skipped
  for (int j = kPre; j < np; ++j)
    acc += wts[j] * *reinterpret_cast<const fcpl*>(parts + j * pstride + 2 + CPL * lane);
  const float inv = den > 0.0f ? 1.0f / den : 0.0f;
  const size_t oq = (size_t)b * p.hkv * G + kvh * G + h;
  *reinterpret_cast<fcpl*>(p.out + oq * D + CPL * lane) = acc * inv;
  if (lane == 0 && p.lse) p.lse[oq] = den > 0.0f ? (M + log2f(den)) * kLn2 : -INFINITY;
}

// TIER: some pages live in the host tier (a separate pool in pinned host memory)
template <int D, int G, bool QBF16, bool TIER>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) void attention_kernel(AttnParams p) {
  __shared__ Smem<D, G> sm;
  // One-dimensional grid, dispatched in index order and spread round-robin
  // over the 8 XCDs. The INT8 regions take `pairs` consecutive items, before
  // (int8_first) or after the INT4 chunks; INT4 item j is chunk j / pairs of
  // pair j % pairs (chunk-major: the first, fullest chunks of every sequence
  // go first, and each XCD gets every 8th pair of every chunk index, i.e. the
  // same mix of sequence lengths). Pair = b * Hkv + kvh. Partial index: INT4
  // chunk j at j, the INT8 region at nsplit.
  const int pairs = p.hkv * p.batch;
  const int n4 = pairs * p.nsplit;
  const int item = blockIdx.x;
  const int i8 = p.int8_first ? item : item - n4;         // INT8 item index if >= 0
  const int i4 = p.int8_first ? item - pairs : item;      // INT4 item index
  int pair, split;
  if (i8 >= 0 && i8 < pairs) {
    pair = i8;
    split = p.nsplit;
  } else {
    pair = i4 % pairs;
    split = i4 / pairs;
  }
  const int kvh = pair % p.hkv, b = pair / p.hkv;
  const int np = p.nsplit + 1;
  float* dst = p.parts + (((size_t)b * p.hkv + kvh) * np + split) * G * (2 + D);
  if (split < p.nsplit) {
    int4_chunk<D, G, QBF16, TIER>(p, sm, b, kvh, split);
    __syncthreads();
    store_partial<D, G>(sm, [&](int w) { return &sm.u.w4[w].ro.o[0][0]; }, dst);
  } else {
    int8_region<D, G, QBF16>(p, sm, b, kvh);
    __syncthreads();
    store_partial<D, G>(sm, [&](int w) { return &sm.u.i8.o[w][0][0]; }, dst);
  }
}

template <int D, int G>
hipError_t launch_dq(const kvc_cache& c, const AttnParams& p, bool qbf16, hipStream_t s) {
  const dim3 grid((unsigned)(p.nsplit + 1) * c.num_kv_heads * c.batch);
  if (p.host_pages > 0) {
    if (qbf16) hipLaunchKernelGGL((attention_kernel<D, G, true, true>), grid, dim3(kThreads), 0, s, p);
    else hipLaunchKernelGGL((attention_kernel<D, G, false, true>), grid, dim3(kThreads), 0, s, p);
  } else {
    if (qbf16) hipLaunchKernelGGL((attention_kernel<D, G, true, false>), grid, dim3(kThreads), 0, s, p);
    else hipLaunchKernelGGL((attention_kernel<D, G, false, false>), grid, dim3(kThreads), 0, s, p);
  }
  hipLaunchKernelGGL((merge_kernel<D, G>), dim3(G, c.num_kv_heads, c.batch), dim3(64), 0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_merge(const float* parts, int parts_per_pair, int batch, int hkv, int G, int D,
                        float* out, float* lse, hipStream_t s) {
  AttnParams p{};
  p.parts = const_cast<float*>(parts);
  p.nsplit = parts_per_pair - 1;
  p.hkv = hkv;
  p.batch = batch;
  p.out = out;
  p.lse = lse;
  const dim3 grid(G, hkv, batch), block(64);
  if (D == 128) {
    switch (G) {
      case 1: hipLaunchKernelGGL((merge_kernel<128, 1>), grid, block, 0, s, p); break;
      case 2: hipLaunchKernelGGL((merge_kernel<128, 2>), grid, block, 0, s, p); break;
      case 4: hipLaunchKernelGGL((merge_kernel<128, 4>), grid, block, 0, s, p); break;
      default: return hipErrorInvalidValue;
    }
  } else {
    switch (G) {
      case 1: hipLaunchKernelGGL((merge_kernel<64, 1>), grid, block, 0, s, p); break;
      case 2: hipLaunchKernelGGL((merge_kernel<64, 2>), grid, block, 0, s, p); break;
      case 4: hipLaunchKernelGGL((merge_kernel<64, 4>), grid, block, 0, s, p); break;
      default: return hipErrorInvalidValue;
    }
  }
  return hipGetLastError();
}

hipError_t launch_attention(const kvc_cache& c, const void* q, kvc_dtype q_dtype, int num_q_heads,
                            float softmax_scale, float* out, float* lse, float* ws,
                            const AttnPlan& plan, int window, hipStream_t s) {
  AttnParams p;
  p.window = window;
  p.sink = c.n_sink;
  p.recent = c.n_recent;
  p.codes_h = c.int4_codes_host;
  p.meta_h = c.int4_meta_host;
  p.host_pages = c.num_host_pages;
  p.q = q;
  p.codes = c.int4_codes;
  p.meta = c.int4_meta;
  p.codes8 = c.int8_codes;
  p.scales8 = c.int8_scales;
  p.block_table = c.block_table;
  p.seq_lens = c.seq_lens;
  p.mask = c.keep_mask;
  p.parts = ws;
  p.out = out;
  p.lse = lse;
  p.alpha = softmax_scale * kLog2e;
  p.hkv = c.num_kv_heads;
  p.batch = c.batch;
  p.max_pages = c.max_pages_per_seq;
  p.num_pages = c.num_phys_pages;
  p.max_ctx = c.max_ctx;
  p.words = mask_words(c.max_ctx);
  p.chunk = plan.chunk;
  p.nsplit = plan.nsplit;
  p.int8_first = plan.int8_first;
  const int G = num_q_heads / c.num_kv_heads;
  const bool bf = q_dtype == KVC_BF16;
  if (c.head_dim == 128) {
    switch (G) {
      case 1: return launch_dq<128, 1>(c, p, bf, s);
      case 2: return launch_dq<128, 2>(c, p, bf, s);
      case 4: return launch_dq<128, 4>(c, p, bf, s);
    }
  } else {
    switch (G) {
      case 1: return launch_dq<64, 1>(c, p, bf, s);
      case 2: return launch_dq<64, 2>(c, p, bf, s);
      case 4: return launch_dq<64, 4>(c, p, bf, s);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace kvc
