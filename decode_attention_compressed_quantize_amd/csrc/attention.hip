// Split-region decode attention over the compressed cache, with the exact
// log-sum-exp merge of the per-chunk partials: in a second, small launch
// (mask mode), in the same launch by the last workgroup of each (sequence,
// kv head) (pool mode), or, with one chunk per pair, by the chunk's own
// workgroup, which then also does the INT8 region (pool mode, fuse8).
//
// Source: KV4-RL review, section 3 - the INT4 region and the protected INT8
// region are processed independently and their outputs are combined by an
// exact softmax merge, so the full-precision cache is never rebuilt; the
// protected region uses high-fidelity probability-value arithmetic, read here
// as float32 P and float32 decoded V.
//
// Work decomposition: one workgroup (4 waves) per INT4 chunk and one per
// (sequence, kv head) for the INT8 region. Every workgroup writes one
// unnormalised partial (m, l, o[D]) per query head: m is the max logit in log2
// units (logit * log2 e), l = sum 2^(s - m), o = sum 2^(s - m) * v. The merge
// combines the partials of each (sequence, kv head) in a fixed order, so
// results do not depend on scheduling. The INT4 records come either from
// the paged store through the keep mask (mask mode: chunk j of a (sequence,
// kv head) is a range of positions whose kept records are gathered), or from
// the kept-record pool (pool mode: chunk j is the j-th of nsplit equal shares
// of that pool's record count, read as contiguous tiles).
//
// INT4 tile of 32 tokens, per wave, in two steps:
//  * K step, logits on v_mfma_f32_16x16x32_f16. A code nibble enters as the
//    exact fp16 subnormal c * 2^-24 (low nibble of a half) or c * 2^-20 (the
//    next nibble), one AND per two values; one MFMA row is one token, one
//    column one (group, head) pair, and the query operand (q scaled per head
//    by a power of two into fp16's top binade, divided by 16 in the slots of
//    second nibbles, zero outside the column's group) makes each column one
//    group's dot product, exact up to float32 accumulation. A float32 query
//    enters as two fp16 parts (two MFMAs). Scale and min are then applied in
//    float32:  s = sum_g scale_g (q_g . c_g) + min_g sum(q_g).
//    The group columns of a head are summed (rotations from the widest, so
//    every column of a head holds the same bits), the running max per head
//    rises when the tile's max does (then the accumulators are rescaled), and
//    each lane takes p = 2^(s - max) of the eight (token, head) pairs its
//    rows hold - exactly the P entries its lanes feed to the V step.
//  * V step, P.V on the same MFMA: rows are (group, head) pairs, columns
//    channels 8n + m of V-code dword n; the P operand is p * V_scale as two
//    fp16 parts, the second scaled by 2^11 into its own accumulator (so
//    probabilities far below fp16's range still count); codes enter as exact
//    fp16 subnormals. Only rows whose group matches the column's channel
//    group are kept. sum_t p_t V_min is accumulated in float32.
#include "kvc_internal.h"
#include "pool_layout.h"

#include <type_traits>

namespace kvc {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kRing = 4;      // INT4 steps in flight per wave (the one in use plus three prefetched)
constexpr float kLoScale = 2048.0f;  // the second fp16 part of P, scaled up by 2^11
#ifndef KVC_POOL_LOAD_AUX
#define KVC_POOL_LOAD_AUX 2
#endif
// cache policy of the pool's direct-to-LDS loads: 2 marks them non-temporal (each
// record is read once per call, so it should not displace reused lines)
constexpr int kLoadAux = KVC_POOL_LOAD_AUX;
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
  float* parts;
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
  // pool mode
  const uint8_t* pool;
  int32_t* pool_header;  // word 3 of a pair's header: its finished workgroups (pool mode)
  int pool_cap;
  uint32_t* errors;
};

__device__ inline void flag(const AttnParams& p, uint32_t bit) {
  if (p.errors) __hip_atomic_fetch_or(p.errors, bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ inline int clamp_len(const AttnParams& p, int L) {
  return L < 0 ? 0 : (L > p.max_ctx ? p.max_ctx : L);
}

// Words at a workgroup-uniform address read through the scalar cache and
// waited for in the same block: the wait counts only scalar and LDS
// operations, so the vector loads already in flight are not waited for (as
// they would be for a vector load issued after them). The words must not
// change during the launch.
__device__ inline uint32_t scalar_load1(const void* ptr) {
  uint32_t v;
  asm volatile("s_load_dword %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(ptr) : "memory");
  return v;
}
// four words at a and one at b, both in flight together
__device__ inline void scalar_load4_1(const void* a, const void* b, u32x4& va, uint32_t& vb) {
  asm volatile("s_load_dwordx4 %0, %2, 0x0\n\ts_load_dword %1, %3, 0x0\n\ts_waitcnt lgkmcnt(0)"
               : "=&s"(va), "=&s"(vb)
               : "s"(a), "s"(b)
               : "memory");
}

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

__device__ inline float2v unpack_f16x2(uint32_t u) {
  return __builtin_convertvector(__builtin_bit_cast(half2v, u), float2v);
}

__device__ inline float4v mfma16x16x32(half8 a, half8 b, float4v c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
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

// 2^e as a float for -126 <= e <= 127.
__device__ inline float exp2i(int e) { return __uint_as_float((uint32_t)(e + 127) << 23); }

template <int D, int G>
struct Shape {
  static constexpr int NG = D / 32;   // quantisation groups per row = QK MFMAs per 16 tokens
  static constexpr int SB = D / 8;    // K-code bytes held per lane slot
  static constexpr int VD = D / 8;    // V-code dwords per token
  static constexpr int NC = NG * G;   // distinct (group, head) columns, <= 16
  static constexpr int MH = NG / 2;   // meta dwords per half row (mask mode staging)
};

// LDS of one workgroup. Mask mode gives each wave its own region (kept list -
// later reused for the wave's output - and staging for one step's V codes
// and meta); pool mode needs only the outputs; the INT8 path overlays its own.
template <int D, int G>
struct Smem {
  static constexpr int kListCap = kMaxChunk / kWaves;  // positions per wave
  static constexpr int kVStride = D / 8 + 4;           // V-code row stride (dwords)
  struct Wave4 {
    union {
      uint32_t rec[kListCap + 32];        // token-record indices, padded with copies
      float o[G][D];                      // the wave's unnormalised output (after the list)
    } ro;
    uint32_t vbuf[32][kVStride];          // V codes of the current 32 tokens
    uint32_t mbuf[32][D / 32];            // K or V (scale | min << 16) of the current 32 tokens
  };
  // INT8 region: the 144 slots' rows (K codes then V codes) at a padded
  // stride, so that 16 rows read at one offset fall in distinct banks
  static constexpr int kRow8 = 2 * D + 16;
  struct Int8 {
    uint8_t rows[144][kRow8];
    float scales[144][2];
    float o[kWaves][G][D];
  };
  // pool mode: each wave's ring of kStage tiles (5 KB: with two workgroups per
  // CU about 10 MB are in flight, where HBM streams fastest; deeper rings read
  // slower) filled by direct-to-LDS loads; after its last tile the wave's
  // output o[G][D] goes to the start of its ring
  static constexpr int kStage = 5120 / (40 * D);
  // a chunk workgroup that also does the INT8 region: the ring, then each
  // wave's (up to) three INT8 blocks of 16 rows and their scales
  static constexpr int kBlk8 = (16 * kRow8 + 128 + 15) / 16 * 16;
  struct Fused8 {
    uint8_t stage[kWaves][kStage][40 * D];
    uint8_t blk[kWaves][3][kBlk8];
  };
  union {
    Wave4 w4[kWaves];
    Int8 i8;
    uint8_t stage[kWaves][kStage][40 * D];
    Fused8 f8;
  } u;
  float m[kWaves][G];
  float l[kWaves][G];
  float vm[kWaves][16];
  float m8[kWaves][G];  // the INT8 part of a chunk workgroup that does both regions
  float l8[kWaves][G];
};

// A store that is performed at device scope (written through this XCD's L2),
// or a plain store.
template <bool COHERENT>
__device__ inline void put_f32(float* a, float v) {
  if constexpr (COHERENT) __hip_atomic_store(a, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else *a = v;
}

// Combine the four waves' (m, l, o) held in LDS into one partial and store it
// (COHERENT: with device-scope stores, for a merge inside the same launch).
// One element (head h, channel ch) of the four waves' combined (M, o, l).
template <int D, int G, typename OF>
__device__ inline void combine_waves(const Smem<D, G>& sm, OF o_of, int h, int ch, float& M, float& o, float& l) {
  M = -INFINITY;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sm.m[w][h]);
  o = 0.0f;
  l = 0.0f;
  if (M != -INFINITY) {
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float mw = sm.m[w][h];
      if (mw == -INFINITY) continue;
      const float a = __builtin_amdgcn_exp2f(mw - M);
      o = __builtin_fmaf(a, o_of(w)[h * D + ch], o);
      l = __builtin_fmaf(a, sm.l[w][h], l);
    }
  }
}

template <int D, int G, bool COHERENT, typename OF>
__device__ inline void store_partial(Smem<D, G>& sm, OF o_of, float* dst) {
  const int tid = threadIdx.x;
  for (int i = tid; i < G * D; i += kThreads) {
    const int h = i / D, ch = i % D;
    float M, o, l;
    combine_waves<D, G>(sm, o_of, h, ch, M, o, l);
    float* row = dst + (size_t)h * (2 + D);
    put_f32<COHERENT>(row + 2 + ch, o);
    if (ch == 0) {
      put_f32<COHERENT>(row, M);
      put_f32<COHERENT>(row + 1, l);
    }
  }
}

// The output of a workgroup that did a pair's whole attention (one chunk per
// pair, INT8 region included): the four waves' INT4 and INT8 (m, l, o)
// combined as in the merge, normalised and stored, with the natural-log lse.
template <int D, int G, typename OF4, typename OF8>
__device__ inline void store_final(const AttnParams& p, Smem<D, G>& sm, OF4 o4_of, OF8 o8_of, int b, int kvh) {
  const int tid = threadIdx.x;
  for (int i = tid; i < G * D; i += kThreads) {
    const int h = i / D, ch = i % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, fmaxf(sm.m[w][h], sm.m8[w][h]));
    float o = 0.0f, l = 0.0f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float mw = sm.m[w][h];
        if (mw == -INFINITY) continue;
        const float a = __builtin_amdgcn_exp2f(mw - M);
        o += a * o4_of(w)[h * D + ch];
        l += a * sm.l[w][h];
      }
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float mw = sm.m8[w][h];
        if (mw == -INFINITY) continue;
        const float a = __builtin_amdgcn_exp2f(mw - M);
        o += a * o8_of(w)[h * D + ch];
        l += a * sm.l8[w][h];
      }
    }
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
    const size_t oq = (size_t)b * p.hkv * G + kvh * G + h;
    p.out[oq * D + ch] = o * inv;
    if (ch == 0 && p.lse) p.lse[oq] = l > 0.0f ? (M + log2f(l)) * kLn2 : -INFINITY;
  }
}

// ------------------------------------------------------------------ INT4 core
// The per-wave state of the INT4 region and the two steps of a 32-token tile.
// Lane (s, n), s = lane / 16, n = lane % 16: column n is (group gc, head hc);
// the lane's C rows, and its P entries, are the tokens tok(i) = 4s + i
// (i < 4) and 16 + 4s + (i - 4) (i >= 4) of the tile.
template <int D, int G, bool QF32>
struct Int4Core {
  using S = Shape<D, G>;
  static constexpr int NG = S::NG, VD = S::VD, NC = S::NC;
  int lane, s, n, gc, hc, vdw;
  float m_col, l_col, vm1;
  float alpha_h;  // softmax scale * log2 e / 2^(e - 24) for the column's head
  float qsp;      // sum of the column's group of q, times 2^(e - 24)
  half8 bqh[NG];
  half8 bql[QF32 ? NG : 1];
  float4v acc[8], accl[8];

  __device__ int tok(int i) const { return i < 4 ? 4 * s + i : 16 + 4 * s + (i - 4); }

  // Query operands of column (gc, hc): entries s*D/4 + 8m + perm[r] of the
  // head (only the slot of group gc is non-zero), scaled by 2^e with e chosen
  // per head so that the largest |q| lands in [2^14, 2^15).
  // The lane's raw query words (bf16 pairs or floats): D/4 entries of its
  // column's head, loaded by load_q so that the loads can be issued early.
  static constexpr int NE = D / 4;
  template <bool QBF16>
  using QRaw = u32x4[QBF16 ? NE / 8 : NE / 4];

  template <bool QBF16>
  __device__ void load_q(const AttnParams& p, int b, int kvh, QRaw<QBF16>& raw) const {
    const int ln = threadIdx.x & 63;
    const size_t qoff = ((size_t)b * p.hkv * G + kvh * G + (ln & 15) % G) * D + (ln >> 4) * NE;
    const u32x4* qp = QBF16 ? reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(p.q) + qoff)
                            : reinterpret_cast<const u32x4*>(reinterpret_cast<const float*>(p.q) + qoff);
#pragma unroll
    for (int i = 0; i < (QBF16 ? NE / 8 : NE / 4); ++i) raw[i] = qp[i];
  }

  template <bool QBF16>
  __device__ void setup(const AttnParams& p, int b, int kvh) {
    QRaw<QBF16> raw;
    load_q<QBF16>(p, b, kvh, raw);
    setup_from<QBF16>(p, raw);
  }

  template <bool QBF16>
  __device__ void setup_from(const AttnParams& p, const QRaw<QBF16>& raw) {
    lane = threadIdx.x & 63;
    s = lane >> 4;
    n = lane & 15;
    gc = (n / G) % NG;
    hc = n % G;
    vdw = n % VD;
    m_col = -INFINITY;
    l_col = vm1 = 0.0f;
#pragma unroll
    for (int m = 0; m < 8; ++m) acc[m] = accl[m] = float4v{0.0f, 0.0f, 0.0f, 0.0f};
    float qe[NE];
    if constexpr (QBF16) {
#pragma unroll
      for (int i = 0; i < NE / 8; ++i) {
        const u32x4 x = raw[i];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          qe[8 * i + 2 * k] = __uint_as_float(x[k] << 16);
          qe[8 * i + 2 * k + 1] = __uint_as_float(x[k] & 0xFFFF0000u);
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < NE / 4; ++i) {
        const u32x4 x = raw[i];
#pragma unroll
        for (int k = 0; k < 4; ++k) qe[4 * i + k] = __uint_as_float(x[k]);
      }
    }
    // the head's largest magnitude (its D entries are spread over the four rows)
    float mx = 0.0f;
#pragma unroll
    for (int i = 0; i < NE; ++i) mx = fmaxf(mx, fabsf(qe[i]));
    mx = rows_max(mx);
    int e = 0;
    if (mx > 0.0f) {
      const int ex = (int)((__float_as_uint(mx) >> 23) & 255u) - 127;  // floor(log2 mx) for normal mx
      e = 14 - ex;
      e = e < -100 ? -100 : (e > 100 ? 100 : e);
    }
    const float qsc = exp2i(e);
    alpha_h = p.alpha * exp2i(24 - e);
    const int slot_group = (s * D / 4) / 32;
    const bool active = slot_group == gc;
    const int perm[8] = {0, 4, 1, 5, 2, 6, 3, 7};
    float qs = 0.0f;
#pragma unroll
    for (int m = 0; m < NG; ++m) {
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const bool x16 = (r == 2 || r == 3 || r == 6 || r == 7);
        const float qv = active ? qe[8 * m + perm[r]] : 0.0f;
        qs += qv;
        const float v = qv * qsc * (x16 ? 0.0625f : 1.0f);  // powers of two: exact
        const _Float16 hi = (_Float16)v;
        bqh[m][r] = hi;
        if constexpr (QF32) bql[m][r] = (_Float16)(v - (float)hi);
      }
    }
    // every entry of the column's group sits in exactly one active slot
    qsp = rows_sum(qs) * exp2i(e - 24);
  }

  // K step: logits of the tile, running max, p of the lane's eight tokens.
  // Tokens at or past lim are not attended (their logits are set to -inf).
  __device__ void k_step(const uint32_t (&kc0)[NG], const uint32_t (&kc1)[NG], const uint32_t (&km)[8],
                         int lim, float (&pr)[8]) {
    float4v c0 = {0.0f, 0.0f, 0.0f, 0.0f}, c1 = c0;
#pragma unroll
    for (int m = 0; m < NG; ++m) {
      uint32_t x = kc0[m];
      uint32_t y = x >> 8;
      half8 a = as_half8(x & 0x000F000Fu, x & 0x00F000F0u, y & 0x000F000Fu, y & 0x00F000F0u);
      c0 = mfma16x16x32(a, bqh[m], c0);
      if constexpr (QF32) c0 = mfma16x16x32(a, bql[m], c0);
      x = kc1[m];
      y = x >> 8;
      a = as_half8(x & 0x000F000Fu, x & 0x00F000F0u, y & 0x000F000Fu, y & 0x00F000F0u);
      c1 = mfma16x16x32(a, bqh[m], c1);
      if constexpr (QF32) c1 = mfma16x16x32(a, bql[m], c1);
    }
    // u_g = scale_g (q_g . c_g) + min_g sum(q_g), both scaled by 2^(e - 24)
    float sv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float d = i < 4 ? c0[i] : c1[i - 4];
      sv[i] = fmaf(h2f(km[i] & 0xFFFFu), d, fmaf(h2f(km[i] >> 16), qsp, 0.0f));
    }
    // sum the group columns of each head, widest rotation first: columns
    // repeat with period NC, so each step adds a pair (x, y) on one lane and
    // (y, x) on its partner, and every column of a head ends with equal bits
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if constexpr (NC >= 8 * G) sv[i] += row_ror<4 * G>(sv[i]);
      if constexpr (NC >= 4 * G) sv[i] += row_ror<2 * G>(sv[i]);
      if constexpr (NC >= 2 * G) sv[i] += row_ror<G>(sv[i]);
    }
    if (__builtin_expect(lim < 32, 0)) {
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (tok(i) >= lim) sv[i] = -INFINITY;
    }
    float tmax = sv[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) tmax = fmaxf(tmax, sv[i]);
    const float mnew = fmaxf(m_col, alpha_h * rows_max(tmax));
    if (__builtin_expect(__ballot(mnew > m_col) != 0, 0)) {
      const float f = __builtin_amdgcn_exp2f(m_col - mnew);  // 0 on the first tile
      l_col *= f;
      vm1 *= f;
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
        for (int m = 0; m < 8; ++m) {
          acc[m][j] *= fj;
          accl[m][j] *= fj;
        }
      }
      m_col = mnew;
    }
    const float mc = m_col == -INFINITY ? 0.0f : m_col;
    float lsum = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      pr[i] = __builtin_amdgcn_exp2f(fmaf(alpha_h, sv[i], -mc));
      lsum += pr[i];
    }
    l_col += lsum;
  }

  // V step: P.V of the tile. vm holds the V meta of group gc of the lane's
  // tokens; for tokens at or past lim it is replaced by zeros (p is 0 there,
  // and the stored meta of such a slot may be anything).
  __device__ void v_step(const uint32_t (&vc)[8], const uint32_t (&vmi)[8], const float (&pr)[8],
                         int lim) {
    uint32_t vm[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) vm[i] = vmi[i];
    if (__builtin_expect(lim < 32, 0)) {
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (tok(i) >= lim) vm[i] = 0u;
    }
    float ps[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      ps[i] = fmaf(pr[i], h2f(vm[i] & 0xFFFFu), 0.0f);
      vm1 = fmaf(pr[i], h2f(vm[i] >> 16), vm1);
    }
    uint32_t ph[4], pl[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      ph[k] = pack_f16x2(ps[2 * k], ps[2 * k + 1]);
      const float2v hf = unpack_f16x2(ph[k]);
      pl[k] = pack_f16x2(fmaf(hf[0], -kLoScale, ps[2 * k] * kLoScale),
                         fmaf(hf[1], -kLoScale, ps[2 * k + 1] * kLoScale));
    }
    const half8 Ah = as_half8(ph[0], ph[1], ph[2], ph[3]);
    const half8 Al = as_half8(pl[0], pl[1], pl[2], pl[3]);
    // V codes of tokens (2q, 2q+1) paired into the halves of one dword
    uint32_t xv[8];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      xv[q] = __builtin_amdgcn_perm(vc[2 * q + 1], vc[2 * q], 0x05040100u);      // channels 0..3
      xv[4 + q] = __builtin_amdgcn_perm(vc[2 * q + 1], vc[2 * q], 0x07060302u);  // channels 4..7
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
      const half8 B = as_half8(bw[0], bw[1], bw[2], bw[3]);
      acc[m] = mfma16x16x32(Ah, B, acc[m]);
      accl[m] = mfma16x16x32(Al, B, accl[m]);
    }
  }

  // The wave's (m, l) per head and its output into LDS (o: [G][D]).
  __device__ void finish(float (&msh)[G], float (&lsh)[G], float (&vmsh)[16], float* o, bool any) {
    if (any) {
      l_col = rows_sum(l_col);  // lane h < G: the sum over the tile rows of head h
      vm1 = rows_sum(vm1);
    }
    if (lane < G) {
      msh[lane] = any ? m_col : -INFINITY;  // lane h < G has column (0, h)
      lsh[lane] = any ? l_col : 0.0f;
    }
    if (lane < 16) vmsh[lane] = vm1;  // side term of row (g, h) = lane g*G + h
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_wave_barrier();
    if (!any) {
      for (int i = lane; i < G * D; i += 64) o[i] = 0.0f;
      return;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = 4 * s + j;
      const int g = (row / G) % NG, h = row % G;
      if (row < NC && g == n / 4 && n < VD) {
        // channel 8n + m: sum p V_scale c, with c entering as c * 2^-24 (m even)
        // or c * 2^-20 (m odd)
        const float side = vmsh[g * G + h];
#pragma unroll
        for (int m = 0; m < 8; ++m) {
          const float v = fmaf(accl[m][j], 1.0f / kLoScale, acc[m][j]);
          o[h * D + 8 * n + m] = fmaf(v, (m & 1) ? 1048576.0f : 16777216.0f, side);
        }
      }
    }
  }
};

// One step's loads: K step = K codes of tokens n and 16 + n (slot s) and meta;
// V step = V codes and meta. Mask mode keeps them raw (meta and V codes are
// transposed through LDS when the step runs); pool mode loads them in the
// core's order (kc0 = w[0..NG), kc1 = w[4..4+NG), meta = w[8..16); V codes
// = w[0..8), V meta = w[8..16)).
struct Step {
  uint32_t w[16];
};

// ------------------------------------------------------------------ INT4, mask mode
// Per wave: compact the kept positions of its quarter of the chunk into an
// LDS list of token-record indices, then walk them in 32-token tiles (a K step
// then a V step each) behind a ring of kRing register steps.
template <int D, int G, bool QBF16, bool TIER>
__device__ void int4_mask_chunk(const AttnParams& p, Smem<D, G>& sm, int b, int kvh, int split) {
  using S = Shape<D, G>;
  constexpr int NG = S::NG, MH = S::MH;
  Int4Core<D, G, !QBF16> core;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int s = lane >> 4;
  const int n = lane & 15;
  const int tl = lane >> 1;  // token this lane stages (compact loads)
  const int hf = lane & 1;   // which half of that token's row
  auto& wv = sm.u.w4[wave];
  int L = p.seq_lens[b];
  if ((L < 0 || L > p.max_ctx) && lane == 0 && wave == 0 && split == 0) flag(p, KVC_ERR_LENGTH);
  L = clamp_len(p, L);
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

  core.template setup<QBF16>(p, b, kvh);

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
    bool bad = false;
    if (pga < 0 || pga >= lim) { bad |= (word & 0x0000FFFFu) != 0; word &= 0xFFFF0000u; }
    if (pgb < 0 || pgb >= lim) { bad |= (word & 0xFFFF0000u) != 0; word &= 0x0000FFFFu; }
    if (__ballot(bad) != 0 && lane == 0) flag(p, KVC_ERR_PAGE);
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
  // per-step guard; padded tokens are not attended (the steps' lim).
  constexpr int kTurn = 16 * kRing;  // tokens per ring turn
  const int padded = (cnt + kTurn - 1) / kTurn * kTurn;
  if (cnt > 0) {
    const uint32_t fill = list[0];
    for (int i = cnt + lane; i < padded; i += 64) list[i] = fill;
  }

  if (cnt > 0) {
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

    // Step 2j brings K codes and K meta of tile j, step 2j + 1 the V codes and
    // V meta of the same tokens. The V half of a token record shares the
    // 128-byte line of its K half, so it is read from L2 right after the K
    // step brought the line in. Both kinds load the same registers with the
    // same instructions (two loads of code dwords, one of meta dwords), so the
    // ring never drains between them. Steps past the end reload the last tile.
    auto fetch = [&](auto kind, int step, Step& t) {
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
        for (int m = 0; m < 4; ++m) { t.w[m] = x[m]; t.w[4 + m] = y[m]; }
        t.w[8] = mm[0];
        t.w[9] = mm[1];
      } else if constexpr (isk) {
        const u32x2 x = *reinterpret_cast<const u32x2*>(a0);
        const u32x2 y = *reinterpret_cast<const u32x2*>(a1);
#pragma unroll
        for (int m = 0; m < 2; ++m) { t.w[m] = x[m]; t.w[4 + m] = y[m]; }
        t.w[8] = *reinterpret_cast<const uint32_t*>(am);
      } else {
        const u32x4 x = *reinterpret_cast<const u32x4*>(a0);
#pragma unroll
        for (int m = 0; m < 4; ++m) t.w[m] = x[m];
        t.w[8] = *reinterpret_cast<const uint32_t*>(am);
      }
    };

    float pr[8];
    // K step: stage the K meta, read the lane's eight (token, group gc) words
    auto kstep = [&](const Step& t, int tile) {
#pragma unroll
      for (int m = 0; m < MH; ++m) wv.mbuf[tl][hf * MH + m] = t.w[8 + m];
      __builtin_amdgcn_wave_barrier();
      uint32_t kc0[NG], kc1[NG], km[8];
#pragma unroll
      for (int m = 0; m < NG; ++m) { kc0[m] = t.w[m]; kc1[m] = t.w[4 + m]; }
#pragma unroll
      for (int i = 0; i < 8; ++i) km[i] = wv.mbuf[core.tok(i)][core.gc];
      __builtin_amdgcn_wave_barrier();
      core.k_step(kc0, kc1, km, cnt - 32 * tile, pr);
    };
    // V step: stage V codes and meta, read the lane's eight dwords of each
    auto vstep = [&](const Step& t, int tile) {
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        if constexpr (D == 128) {
          wv.vbuf[lane >> 2][4 * (lane & 3) + m] = t.w[m];
          wv.vbuf[16 + (lane >> 2)][4 * (lane & 3) + m] = t.w[4 + m];
        } else {
          wv.vbuf[lane >> 1][4 * (lane & 1) + m] = t.w[m];
        }
      }
#pragma unroll
      for (int m = 0; m < MH; ++m) wv.mbuf[tl][hf * MH + m] = t.w[8 + m];
      __builtin_amdgcn_wave_barrier();
      uint32_t vc[8], vm[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        vc[i] = wv.vbuf[core.tok(i)][core.vdw];
        vm[i] = wv.mbuf[core.tok(i)][core.gc];
      }
      __builtin_amdgcn_wave_barrier();
      core.v_step(vc, vm, pr, cnt - 32 * tile);
    };

    // slot j of the ring always holds a step of parity j, so every unrolled
    // slot knows its kind at compile time
    using KStep = std::integral_constant<bool, true>;
    using VStep = std::integral_constant<bool, false>;
    Step ring[kRing];
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
        if (j % 2 == 0) kstep(ring[j], (step + j) >> 1);
        else vstep(ring[j], (step + j) >> 1);
      }
    }
  }
  core.finish(sm.m[wave], sm.l[wave], sm.vm[wave], &wv.ro.o[0][0], cnt > 0);
}

// ------------------------------------------------------------------ INT8 region
// The <= 144 protected positions of one (sequence, kv head): high-fidelity
// attention over INT8 codes (KV4-RL review, sections 1 and 3).
// Which slots hold attended positions follows from L alone: all 144 when
// L >= 144, else exactly slots [0, L) (slot = position below 144). So every
// slot's codes and scales are loaded and masked afterwards.
// The 144 slots form 9 blocks of 16; wave w takes blocks w, w + 4, w + 8
// (those below 9). Where a wave keeps its blocks in LDS is the caller's: a
// workgroup of the INT8 region alone loads them into its Int8 area; a chunk
// workgroup that also does the INT8 region (one chunk per pair) loads them
// into an area of each wave's own beside its ring.
//  - Loads: each slot's K and V rows (2D bytes, at a padded stride so that the
//    16 rows read at one offset fall in distinct banks) and the block's scales
//    go straight to LDS with 4-byte direct-to-LDS loads, one row per
//    instruction, coalesced, and one more for the block's scales.
//  - Logits on v_mfma_f32_16x16x32_f16: rows are 16 slots, columns the G
//    heads. A code c enters as the exact fp16 subnormal (c + 128) * 2^-24 (a
//    byte XOR and a byte permute); the query is scaled per head by a power of
//    two into [2^14, 2^15) and split into two fp16 parts (one for a bf16
//    query), so q.(c + 128) is float32-accurate, and 128 * sum(q) is taken off
//    in float32.
//  - Softmax per head over the wave's slots, then P.V in float32 on the VALU
//    (lane = channels, p * V_scale from LDS, codes read from the rows).
constexpr int kSlots8 = kSink + kRecent;
constexpr int kBlocks8 = kSlots8 / 16;                      // 9
constexpr int kWaveBlocks8 = (kBlocks8 + kWaves - 1) / kWaves;  // 3
static_assert(kSlots8 == 144 && kSlots8 % 16 == 0, "INT8 slots");

template <int D>
constexpr int row8_stride() { return 2 * D + 16; }

// Block rb (< 9) of the INT8 slots starting at slot `base` (pair * 144):
// rows to `rows` (16 x row8_stride bytes), scales to `sc` ([16][2] floats).
template <int D>
__device__ inline void int8_issue_block(const AttnParams& p, size_t base, int rb, uint8_t* rows, float* sc) {
  const int lane = threadIdx.x & 63;
  const uint8_t* src = reinterpret_cast<const uint8_t*>(p.codes8) + (base + 16 * (size_t)rb) * 2 * D;
#pragma unroll
  for (int r = 0; r < 16; ++r)
    if (lane < 2 * D / 4)
      __builtin_amdgcn_global_load_lds(src + r * 2 * D + lane * 4,
                                       (__attribute__((address_space(3))) void*)(rows + r * row8_stride<D>()), 4,
                                       0, 0);
  const uint8_t* ssrc = reinterpret_cast<const uint8_t*>(p.scales8 + (base + 16 * (size_t)rb) * 2);
  if (lane < 32)
    __builtin_amdgcn_global_load_lds(ssrc + lane * 4, (__attribute__((address_space(3))) void*)sc, 4, 0, 0);
}

// The query entries lane (s4, n) needs: head n (< G) at dims 32 kk + 8 s4 + t.
template <int D, int G, bool QBF16>
__device__ inline void int8_load_q(const AttnParams& p, int b, int kvh, float (&qe)[D / 32][8]) {
  const int lane = threadIdx.x & 63;
  const int s4 = lane >> 4, n = lane & 15;
  const int hq = n < G ? n : 0;
  const size_t qoff = ((size_t)b * p.hkv * G + kvh * G + hq) * D;
#pragma unroll
  for (int kk = 0; kk < D / 32; ++kk)
#pragma unroll
    for (int t = 0; t < 8; ++t) qe[kk][t] = load_q<QBF16>(p.q, qoff + 32 * kk + 8 * s4 + t);
}

// The wave's blocks, already in LDS: blk(i, rows, sc) gives block i's rows
// and scales. Out: m and l of column n (lane n < G: head n; base-2 logits),
// and the wave's unnormalised output of head h at o_dst[h * D + channel]
// (LDS; 0 when the wave has no valid slot, and then m = -inf, l = 0).
// Both contractions run on MFMA with the lane layout of a 16 x 16 tile
// (lane (s4, n): column n, rows 4 s4 + j):
//  - logits C[slot][head] over k = the head dimension (16x16x32): A = the
//    slot's K codes, B = the scaled query, hi and lo parts in two
//    accumulators; every block's chain is issued together (a block past the
//    wave's valid ones reads the wave's first block and is masked);
//  - P.V C[channel][head] over k = the block's 16 slots (16x16x16): A = the
//    V codes (code c enters as (c + 128) 2^-24), B = p * V_scale of the
//    lane's own four slots, split into fp16 hi and lo parts accumulated
//    together (float32-accurate), then o = 2^24 C - 128 sum(p * V_scale).
template <int D, int G, bool QBF16, typename BLK>
__device__ inline void int8_wave(const AttnParams& p, int nvalid, const float (&qe)[D / 32][8], BLK blk,
                                 float& m_out, float& l_out, float* o_dst) {
  constexpr int NK = D / 32;  // logit k-steps over the head dimension
  constexpr int NT = D / 16;  // P.V channel tiles
  constexpr int kRow = row8_stride<D>();
  constexpr int NB8 = kWaveBlocks8;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int s4 = lane >> 4, n = lane & 15;
  // ---- query operands of column n (head n < G): 2^e_h * q, hi and lo fp16
  float mx = 0.0f, qsum = 0.0f;
#pragma unroll
  for (int kk = 0; kk < NK; ++kk)
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      mx = fmaxf(mx, fabsf(qe[kk][t]));
      qsum += qe[kk][t];
    }
  mx = rows_max(mx);  // over the head's D entries (four lanes n, n + 16, ...)
  qsum = rows_sum(qsum);
  int e = 0;
  if (mx > 0.0f) {
    const int ex = (int)((__float_as_uint(mx) >> 23) & 255u) - 127;
    e = 14 - ex;
    e = e < -100 ? -100 : (e > 100 ? 100 : e);
  }
  const float qsc = exp2i(e);
  half8 bh[NK], bl[QBF16 ? 1 : NK];
#pragma unroll
  for (int kk = 0; kk < NK; ++kk)
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const float v = n < G ? qe[kk][t] * qsc : 0.0f;
      const _Float16 hi = (_Float16)v;
      bh[kk][t] = hi;
      if constexpr (!QBF16) bl[kk][t] = (_Float16)(v - (float)hi);
    }
  // logit of code sum: (acc * 2^(24 - e) - 128 * sum(q)) * K_scale * alpha
  const float unscale = exp2i(24 - e);
  const float off = 128.0f * qsum;
  // ---- the wave's blocks
  bool vb[NB8];
  int rb[NB8];
  const uint8_t* rows[NB8];
  const float* sc[NB8];
#pragma unroll
  for (int i = 0; i < NB8; ++i) {
    rb[i] = wave + kWaves * i;
    vb[i] = rb[i] < kBlocks8 && 16 * rb[i] < nvalid;
    blk(vb[i] ? i : 0, rows[i], sc[i]);
  }
  // ---- logits
  float4v ch[NB8], cl[NB8];
#pragma unroll
  for (int i = 0; i < NB8; ++i) ch[i] = cl[i] = float4v{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int kk = 0; kk < NK; ++kk)
#pragma unroll
    for (int i = 0; i < NB8; ++i) {
      const uint2 x = *reinterpret_cast<const uint2*>(rows[i] + n * kRow + 32 * kk + 8 * s4);
      const uint32_t x0 = x.x ^ 0x80808080u, x1 = x.y ^ 0x80808080u;
      const half8 a = as_half8(__builtin_amdgcn_perm(0u, x0, 0x0c010c00u), __builtin_amdgcn_perm(0u, x0, 0x0c030c02u),
                               __builtin_amdgcn_perm(0u, x1, 0x0c010c00u), __builtin_amdgcn_perm(0u, x1, 0x0c030c02u));
      ch[i] = mfma16x16x32(a, bh[kk], ch[i]);
      if constexpr (!QBF16) cl[i] = mfma16x16x32(a, bl[kk], cl[i]);
    }
  float sl[NB8][4];
  float m = -INFINITY;
#pragma unroll
  for (int i = 0; i < NB8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int t = 4 * s4 + j;
      const bool valid = vb[i] && 16 * rb[i] + t < nvalid;
      const float acc = QBF16 ? ch[i][j] : ch[i][j] + cl[i][j];
      const float v = (acc * unscale - off) * sc[i][2 * t] * p.alpha;
      sl[i][j] = valid ? v : -INFINITY;
      m = fmaxf(m, sl[i][j]);
    }
  m = rows_max(m);  // over the wave's slots, per head (column n)
  // ---- softmax weights; B operands p * V_scale (column n, slots 4 s4 + j)
  typedef _Float16 half4 __attribute__((ext_vector_type(4)));
  half4 Bh[NB8], Bl[NB8];
  float l = 0.0f, ps = 0.0f;
#pragma unroll
  for (int i = 0; i < NB8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int t = 4 * s4 + j;
      const bool valid = vb[i] && 16 * rb[i] + t < nvalid && n < G;
      // slots past the length may hold anything: their weight is exactly 0
      const float pr = valid ? __builtin_amdgcn_exp2f(sl[i][j] - m) : 0.0f;
      const float pv = valid ? pr * sc[i][2 * t + 1] : 0.0f;
      l += pr;
      ps += pv;
      const _Float16 hi = (_Float16)pv;
      Bh[i][j] = hi;
      Bl[i][j] = (_Float16)(pv - (float)hi);
    }
  l = rows_sum(l);
  ps = rows_sum(ps);
  const bool any = m != -INFINITY;
  // ---- P.V: channel tile c, rows = channels 16 c + 4 s4 + r, column = head n
  float4v oc[NT];
#pragma unroll
  for (int c = 0; c < NT; ++c) oc[c] = float4v{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int i = 0; i < NB8; ++i) {
    if (!vb[i]) continue;
    const uint8_t* vr = rows[i] + D + n;  // lane reads channel 16 c + n of slots 4 s4 + j
#pragma unroll
    for (int c = 0; c < NT; ++c) {
      const uint32_t b0 = vr[(4 * s4 + 0) * kRow + 16 * c], b1 = vr[(4 * s4 + 1) * kRow + 16 * c];
      const uint32_t b2 = vr[(4 * s4 + 2) * kRow + 16 * c], b3 = vr[(4 * s4 + 3) * kRow + 16 * c];
      const uint32_t w0 = (b0 | (b1 << 16)) ^ 0x00800080u, w1 = (b2 | (b3 << 16)) ^ 0x00800080u;
      const half4 A = __builtin_bit_cast(half4, (u32x2){w0, w1});
      oc[c] = __builtin_amdgcn_mfma_f32_16x16x16f16(A, Bh[i], oc[c], 0, 0, 0);
      oc[c] = __builtin_amdgcn_mfma_f32_16x16x16f16(A, Bl[i], oc[c], 0, 0, 0);
    }
  }
  if (n < G) {
#pragma unroll
    for (int c = 0; c < NT; ++c)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        o_dst[n * D + 16 * c + 4 * s4 + r] = any ? fmaf(oc[c][r], 16777216.0f, -128.0f * ps) : 0.0f;
  }
  m_out = any ? m : -INFINITY;
  l_out = any ? l : 0.0f;
}

// ------------------------------------------------------------------ INT4, pool mode
// Reads one staged tile of the lane's pieces from LDS: K codes of tokens n and
// 16 + n (slot s), then for each half h of the lane's eight tokens the K meta
// of group gc, the V-code dword vdw and the V meta of group gc. The wait for
// the tile's direct-to-LDS loads (all but the VMC issued after it) and the LDS
// reads' own completion are inside the one asm block, so no read is in flight
// when it ends; LDS reads of the compiler's would make it wait for every
// outstanding direct-to-LDS load instead.
template <int D, int VMC>
__device__ inline void read_staged(uint32_t lds, uint32_t o_kc, uint32_t o_km, uint32_t o_vc,
                                   uint32_t o_vm, u32x4 (&r)[8]) {
  constexpr int NG = D / 32, VD = D / 8;
  constexpr int KMH = 4 * NG * 16, VCH = 4 * VD * 16;  // byte offset of the second half
  if constexpr (D == 128) {
    asm volatile(
        "s_waitcnt vmcnt(%8)\n\t"
        "ds_read_b128 %0, %9\n\t"
        "ds_read_b128 %1, %9 offset:1024\n\t"
        "ds_read_b128 %2, %10\n\t"
        "ds_read_b128 %3, %10 offset:%11\n\t"
        "ds_read_b128 %4, %12\n\t"
        "ds_read_b128 %5, %12 offset:%13\n\t"
        "ds_read_b128 %6, %14\n\t"
        "ds_read_b128 %7, %14 offset:%11\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]),
          "=&v"(r[7])
        : "n"(VMC), "v"(lds + o_kc), "v"(lds + o_km), "n"(KMH), "v"(lds + o_vc), "n"(VCH),
          "v"(lds + o_vm)
        : "memory");
  } else {
    u32x2 k0, k1;
    asm volatile(
        "s_waitcnt vmcnt(%8)\n\t"
        "ds_read_b64 %0, %9\n\t"
        "ds_read_b64 %1, %9 offset:512\n\t"
        "ds_read_b128 %2, %10\n\t"
        "ds_read_b128 %3, %10 offset:%11\n\t"
        "ds_read_b128 %4, %12\n\t"
        "ds_read_b128 %5, %12 offset:%13\n\t"
        "ds_read_b128 %6, %14\n\t"
        "ds_read_b128 %7, %14 offset:%11\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(k0), "=&v"(k1), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]),
          "=&v"(r[7])
        : "n"(VMC), "v"(lds + o_kc), "v"(lds + o_km), "n"(KMH), "v"(lds + o_vc), "n"(VCH),
          "v"(lds + o_vm)
        : "memory");
    r[0] = u32x4{k0[0], k0[1], 0u, 0u};
    r[1] = u32x4{k1[0], k1[1], 0u, 0u};
  }
}

// read_staged with the wait for `after` tiles of NL loads each still in
// flight behind the one read (at most N; the count is an immediate, so the
// few tail cases are separate instantiations).
template <int D, int NL, int N>
__device__ inline void read_staged_after(int after, uint32_t lds, uint32_t o_kc, uint32_t o_km, uint32_t o_vc,
                                         uint32_t o_vm, u32x4 (&r)[8]) {
  if constexpr (N == 0) {
    read_staged<D, 0>(lds, o_kc, o_km, o_vc, o_vm, r);
  } else {
    if (after >= N) read_staged<D, NL * N>(lds, o_kc, o_km, o_vc, o_vm, r);
    else read_staged_after<D, NL, N - 1>(after, lds, o_kc, o_km, o_vc, o_vm, r);
  }
}

// Chunk `split` of the pool of (b, kvh): records [r0, r1), the split-th of
// nsplit equal shares (whole 32-record tiles) of the pool's count. Tile
// t0 + wave + 4j goes to wave `wave` (the four waves read neighbouring tiles
// at any time). Each wave streams its tiles through a ring of kStage LDS
// buffers filled by direct-to-LDS loads (one 16-byte piece per lane per
// instruction, whole contiguous tiles), so kStage tiles are in flight per
// wave without holding registers; a tile's pieces then come out of LDS in
// the order the core consumes them. The pool header, the query and the first
// tiles (guessed from the capacity, checked against the count) are all
// requested at once, and the query is converted while they are in flight.
template <int D, int G, bool QBF16, bool FUSE8>
__device__ void int4_pool_chunk(const AttnParams& p, Smem<D, G>& sm, int b, int kvh, int split) {
  using S = Shape<D, G>;
  constexpr int NG = S::NG, VD = S::VD;
  constexpr int TILE = 40 * D, KM = 16 * D, VC = 20 * D, VM = 36 * D;
  constexpr int NB = Smem<D, G>::kStage;
  // direct-to-LDS loads per tile and wave: 1 KB pieces (16 bytes a lane), then
  // 256-byte pieces (4 bytes a lane) for the rest of a D = 64 tile
  constexpr int NL16 = TILE / 1024, NL4 = (TILE % 1024) / 256, NL = NL16 + NL4;
  Int4Core<D, G, !QBF16> core;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int pair = b * p.hkv + kvh;
  // the query is loaded first and converted while the first tiles are in flight
  typename Int4Core<D, G, !QBF16>::template QRaw<QBF16> qraw;
  core.template load_q<QBF16>(p, b, kvh, qraw);
  // FUSE8 (one chunk per pair): the workgroup does the INT8 region too. Each
  // wave's blocks are requested now, into LDS of their own beside the ring
  // (before the tiles, so the tiles' waits need not count them), and used
  // after the INT4 loop.
  constexpr int kRow8 = Smem<D, G>::kRow8;
  static_assert(kWaveBlocks8 == 3 && 16 * kRow8 + 128 <= Smem<D, G>::kBlk8 && G * D * 4 <= 3 * Smem<D, G>::kBlk8,
                "INT8 blocks and their output fit the wave's block area");
  const int slots8 = FUSE8 ? p.sink + p.recent : 0;
  if constexpr (FUSE8) {
    if (slots8 > 0) {
      const size_t base8 = ((size_t)b * p.hkv + kvh) * slots8;
#pragma unroll
      for (int i = 0; i < kWaveBlocks8; ++i) {
        const int rb = wave + kWaves * i;
        uint8_t* r = &sm.u.f8.blk[wave][i][0];
        if (rb < kBlocks8) int8_issue_block<D>(p, base8, rb, r, reinterpret_cast<float*>(r + 16 * kRow8));
      }
    }
  }
  // this wave's first tile and tile count for a pool of c records (records [r0, r1))
  auto range = [&](int c, int& t0, int& ntw, int& r1) {
    const int share = ((c + p.nsplit - 1) / p.nsplit + kPoolTile - 1) / kPoolTile * kPoolTile;
    const int r0 = split * share;
    r1 = r0 + share < c ? r0 + share : c;
    const int ntiles = r1 > r0 ? (r1 - r0 + kPoolTile - 1) / kPoolTile : 0;
    t0 = __builtin_amdgcn_readfirstlane(r0 / kPoolTile);
    ntw = __builtin_amdgcn_readfirstlane(ntiles > wave ? (ntiles - wave + kWaves - 1) / kWaves : 0);
  };
  const uint8_t* base = p.pool + (size_t)pair * pool_pair_bytes(D, p.pool_cap);
  uint8_t* ring = &sm.u.stage[wave][0][0];
  const uint32_t ring_lds = (uint32_t)(uintptr_t)ring;
  // direct-to-LDS loads of pool tile `tile` of the pair into ring slot k
  auto issue_tile = [&](int tile, int k) {
    const uint8_t* src = base + (size_t)tile * TILE;
    uint8_t* dst = ring + k * TILE;
#pragma unroll
    for (int i = 0; i < NL16; ++i)
      __builtin_amdgcn_global_load_lds(src + i * 1024 + lane * 16,
                                       (__attribute__((address_space(3))) void*)(dst + i * 1024), 16, 0, kLoadAux);
#pragma unroll
    for (int i = 0; i < NL4; ++i)
      __builtin_amdgcn_global_load_lds(src + NL16 * 1024 + i * 256 + lane * 4,
                                       (__attribute__((address_space(3))) void*)(dst + NL16 * 1024 + i * 256),
                                       4, 0, kLoadAux);
  };
  int t0, ntw, r1;
  // tile jt of this wave into ring slot k
  auto issue = [&](int jt, int k) { issue_tile(t0 + wave + kWaves * jt, k); };
  // The first NB tiles are requested before the header is in, for the chunk
  // a full pool (count = capacity) would give; a count that rounds to the
  // same 32-record shares (always with one chunk per pair, and for a budget
  // near the capacity) keeps them. Exactly NB tiles are requested (a wave
  // with fewer re-reads its first one, or the pair's tile 0), so that the
  // wait for the query loaded before them is exact; every tile lies inside
  // the pool's capacity (64 records or more).
  range(p.pool_cap, t0, ntw, r1);
  const int t0_guess = t0, ntw_guess = ntw;
#pragma unroll
  for (int k = 0; k < NB; ++k)
    issue_tile(k < ntw_guess ? t0 + wave + kWaves * k : (ntw_guess > 0 ? t0 + wave : 0), k);
  // header and length through the scalar cache (word 3, which this launch
  // changes, is not used here)
  u32x4 hdr;
  uint32_t Lw;
  scalar_load4_1(p.pool_header + 4 * (size_t)pair, p.seq_lens + b, hdr, Lw);
  const int L = (int)Lw;
  // the query's conversion (which waits for every load in flight: the tiles'
  // direct-to-LDS loads leave the compiler no exact count) stays behind the
  // header's load
#pragma unroll
  for (auto& x : qraw) asm volatile("" : "+v"(x));
  core.template setup_from<QBF16>(p, qraw);
  int cnt = 0;
  if (hdr[2] == kPoolMagic) {
    cnt = (int)hdr[0];
    cnt = cnt < 0 ? 0 : (cnt > p.pool_cap ? p.pool_cap : cnt);
  }
  // the pool must describe the current length (reported once per pair)
  if (split == 0 && threadIdx.x == 0 && (hdr[2] != kPoolMagic || (int)hdr[1] != clamp_len(p, L)))
    flag(p, KVC_ERR_POOL);
  range(cnt, t0, ntw, r1);
  if (t0 != t0_guess || ntw > ntw_guess) {
    // other tiles: the guessed loads land first, then the ring is refilled
    __builtin_amdgcn_s_waitcnt(0);
#pragma unroll
    for (int k = 0; k < NB; ++k)
      if (k < ntw) issue(k, k);
  }
  // else: the same tiles. Slots past ntw hold tiles that are never read: the
  // per-tile waits below count only the tiles < ntw issued after a tile, at
  // most what is in flight behind it, so they only wait longer.
  if (FUSE8 && threadIdx.x == 0 && (L < 0 || L > p.max_ctx)) flag(p, KVC_ERR_LENGTH);
  // FUSE8: the wave's INT8 part (its blocks are in LDS since before the first
  // tile). It runs inside the INT4 loop, before tile s8 of the wave is read
  // (the tiles in flight land meanwhile); s8 differs from wave to wave, so that across the chip the INT8 parts are
  // spread over the streaming instead of all running after it, when the HBM
  // would have nothing to do. A wave without INT4 tiles does it after the loop.
  float m8 = -INFINITY, l8 = 0.0f;
  float* o8d = reinterpret_cast<float*>(&sm.u.f8.blk[wave][0][0]);  // after the blocks are read
  auto int8_part = [&] {
    if constexpr (FUSE8) {
      if (slots8 > 0) {
        const int Lc = clamp_len(p, L);
        const int nvalid = Lc < slots8 ? Lc : slots8;
        float qe[D / 32][8];
        int8_load_q<D, G, QBF16>(p, b, kvh, qe);
        __builtin_amdgcn_s_waitcnt(0);  // the wave's blocks and its query are in
        int8_wave<D, G, QBF16>(
            p, nvalid, qe,
            [&](int i, const uint8_t*& rows, const float*& sc) {
              rows = &sm.u.f8.blk[wave][i][0];
              sc = reinterpret_cast<const float*>(rows + 16 * kRow8);
            },
            m8, l8, o8d);
      } else {
        for (int i = lane; i < G * D; i += 64) o8d[i] = 0.0f;
      }
    }
  };
  const int s8 = ntw > 0 ? __builtin_amdgcn_readfirstlane((int)((blockIdx.x * kWaves + wave) % ntw)) : -1;
  if (ntw > 0) {
    const int s = lane >> 4;
    const uint32_t o_kc = (uint32_t)lane * S::SB;
    const uint32_t o_km = KM + (s * NG + core.gc) * 16;
    const uint32_t o_vc = VC + (s * VD + core.vdw) * 16;
    const uint32_t o_vm = VM + (s * NG + core.gc) * 16;
    float pr[8];
    for (int jt0 = 0; jt0 < ntw; jt0 += NB) {
#pragma unroll 1
      for (int k = 0; k < NB; ++k) {
        const int jt = jt0 + k;
        if (jt >= ntw) break;
        u32x4 r[8];
        // tiles in flight behind this one: NB - 1, fewer at the end (no tile
        // is loaded twice)
        if (FUSE8 && __builtin_expect(jt == s8, 0)) int8_part();
        read_staged_after<D, NL, NB - 1>(ntw - 1 - jt, ring_lds + k * TILE, o_kc, o_km, o_vc, o_vm, r);
        if (jt + NB < ntw) issue(jt + NB, k);
        const int lim = r1 - 32 * (t0 + wave + kWaves * jt);
        uint32_t kc0[NG], kc1[NG], km[8], vc[8], vm[8];
#pragma unroll
        for (int m = 0; m < NG; ++m) { kc0[m] = r[0][m]; kc1[m] = r[1][m]; }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          km[i] = r[2][i]; km[4 + i] = r[3][i];
          vc[i] = r[4][i]; vc[4 + i] = r[5][i];
          vm[i] = r[6][i]; vm[4 + i] = r[7][i];
        }
        core.k_step(kc0, kc1, km, lim, pr);
        core.v_step(vc, vm, pr, lim);
      }
    }
  }
  if (FUSE8 && ntw <= 0) int8_part();
  // the wave's output goes to the start of its own ring (its loads are done
  // first; with FUSE8 the INT8 part has read its blocks)
  __builtin_amdgcn_s_waitcnt(0);
  core.finish(sm.m[wave], sm.l[wave], sm.vm[wave], reinterpret_cast<float*>(&sm.u.stage[wave][0][0]),
              ntw > 0);
  if constexpr (FUSE8) {
    // the INT8 part's (m, l) beside the INT4 ones (its o is in the block area)
    if (lane < G) {  // lane h holds column h
      sm.m8[wave][lane] = m8;
      sm.l8[wave][lane] = l8;
    }
  }
}

// ------------------------------------------------------------------ INT8 region workgroup
// The INT8 region of one (sequence, kv head) in a workgroup of its own: each
// wave loads its blocks into the Int8 area, then does its part (int8_wave).
// The wave's (m, l, o) per head go to LDS for store_partial.
// after_loads() runs in every thread once the wave's blocks are in (it may
// synchronise the workgroup).
template <int D, int G, bool QBF16, typename AL>
__device__ void int8_region(const AttnParams& p, Smem<D, G>& sm, int b, int kvh, AL after_loads) {
  static_assert(Smem<D, G>::kRow8 == row8_stride<D>(), "INT8 row stride");
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int slots = p.sink + p.recent;  // 144, or 0 without INT8 protection
  auto& i8 = sm.u.i8;
  // rows and scales of every slot, requested without waiting for the length
  // (slots past it are masked, whatever they hold)
  const size_t base = ((size_t)b * p.hkv + kvh) * slots;
  if (slots > 0) {
#pragma unroll
    for (int i = 0; i < kWaveBlocks8; ++i) {
      const int rb = wave + kWaves * i;
      if (rb < kBlocks8) int8_issue_block<D>(p, base, rb, &i8.rows[16 * rb][0], &i8.scales[16 * rb][0]);
    }
  }
  float qe[D / 32][8];
  int8_load_q<D, G, QBF16>(p, b, kvh, qe);
  // the length, read after the loads above are issued
  int L = (int)scalar_load1(p.seq_lens + b);
  if ((L < 0 || L > p.max_ctx) && threadIdx.x == 0) flag(p, KVC_ERR_LENGTH);
  L = clamp_len(p, L);
  const int nvalid = L < slots ? L : slots;
  __builtin_amdgcn_s_waitcnt(0);  // the wave's own blocks are in
  after_loads();
  float m, l;
  int8_wave<D, G, QBF16>(
      p, nvalid, qe,
      [&](int i, const uint8_t*& rows, const float*& sc) {
        const int rb = wave + kWaves * i;
        rows = &i8.rows[16 * rb][0];
        sc = &i8.scales[16 * rb][0];
      },
      m, l, &i8.o[wave][0][0]);
  if (lane < G) {  // lane h holds column h
    sm.m[wave][lane] = m;
    sm.l[wave][lane] = l;
  }
}

// ------------------------------------------------------------------ merge
// One wave merges the nsplit + 1 partials of one (sequence, kv head) for one
// query head in a fixed order (outputs summed in index order):
// M = max_j m_j, w_j = 2^(m_j - M) (0 for empty partials),
// out = sum_j w_j o_j / sum_j w_j l_j, lse = ln 2 * (M + log2 sum_j w_j l_j).
// Lane l owns output channels [l*CPL, l*CPL + CPL); the (m, l) pairs and the
// lane's slices of the first kPre partials are loaded together up front.
// wts: kMaxParts floats of LDS that only this wave uses. COHERENT: the
// partials were written in the same launch with device-scope stores, so they
// are read with device-scope loads (past this XCD's L2).
template <int D, int G, bool COHERENT>
__device__ void merge_head(const AttnParams& p, int b, int kvh, int h, int lane, float* wts) {
  constexpr int CPL = D / 64;  // channels per lane
  constexpr int kPre = 32;     // partials whose slices are loaded up front
  typedef float fcpl __attribute__((ext_vector_type(CPL)));
  // CPL (1 or 2) consecutive floats, as one load
  auto ld = [](const float* a) -> fcpl {
    if constexpr (!COHERENT) {
      return *reinterpret_cast<const fcpl*>(a);
    } else if constexpr (CPL == 2) {
      const uint64_t u = __hip_atomic_load(reinterpret_cast<const uint64_t*>(a), __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
      return __builtin_bit_cast(fcpl, u);
    } else {
      const float v = __hip_atomic_load(a, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return __builtin_bit_cast(fcpl, v);
    }
  };
  auto ld2 = [](const float* a) -> float2v {
    if constexpr (!COHERENT) {
      return *reinterpret_cast<const float2v*>(a);
    } else {
      const uint64_t u = __hip_atomic_load(reinterpret_cast<const uint64_t*>(a), __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
      return __builtin_bit_cast(float2v, u);
    }
  };
  const int np = p.nsplit + 1;
  const size_t pstride = (size_t)G * (2 + D);
  const float* run = p.parts + ((size_t)b * p.hkv + kvh) * np * pstride + (size_t)h * (2 + D);
  auto part = [&](int j) -> const float* { return run + (size_t)j * pstride; };
  fcpl pre[kPre];
#pragma unroll
  for (int j = 0; j < kPre; ++j) {
    const int jj = j < np ? j : np - 1;
    pre[j] = ld(part(jj) + 2 + CPL * lane);
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
      const float2v ml = ld2(part(j));
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
    den = __builtin_fmaf(w, lj[r], den);
    if (j < np) wts[j] = w;
  }
  den = wave_sum(den);
  __builtin_amdgcn_wave_barrier();  // one wave: its LDS writes are seen by its later reads
  // acc = sum_j w_j o_j as fused multiply-adds in index order (the two-partial
  // shortcut of the INT8 workgroup repeats exactly these operations)
  fcpl acc = {};
  auto fma_acc = [&](float w, fcpl v) {
#pragma unroll
    for (int c = 0; c < CPL; ++c) acc[c] = __builtin_fmaf(w, v[c], acc[c]);
  };
#pragma unroll
  for (int j = 0; j < kPre; ++j)
    if (j < np) fma_acc(wts[j], pre[j]);
  // every partial is written by the attention kernel, so no load is skipped
  for (int j = kPre; j < np; ++j) fma_acc(wts[j], ld(part(j) + 2 + CPL * lane));
  const float inv = den > 0.0f ? 1.0f / den : 0.0f;
  const size_t oq = (size_t)b * p.hkv * G + kvh * G + h;
  *reinterpret_cast<fcpl*>(p.out + oq * D + CPL * lane) = acc * inv;
  if (lane == 0 && p.lse) p.lse[oq] = den > 0.0f ? (M + log2f(den)) * kLn2 : -INFINITY;
}

// One wave per (query head, kv head, sequence).
template <int D, int G>
__global__ __launch_bounds__(64) void merge_kernel(AttnParams p) {
  __shared__ float wts[kMaxParts];
  merge_head<D, G, false>(p, blockIdx.z, blockIdx.y, blockIdx.x, threadIdx.x, wts);
}

// TIER: some pages live in the host tier (a separate pool in pinned host memory).
// POOL: the INT4 records come from the kept-record pool.
// FUSE8 (pool mode, one chunk per pair): workgroup = pair, which does the
// INT8 region too and writes the output itself (no partials, no merge).
template <int D, int G, bool QBF16, bool TIER, bool POOL, bool FUSE8>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) void attention_kernel(AttnParams p) {
  __shared__ Smem<D, G> sm;
  if constexpr (FUSE8) {
    static_assert(POOL, "FUSE8 is a pool mode");
    const int pair = blockIdx.x;
    const int kvh = pair % p.hkv, b = pair / p.hkv;
    int4_pool_chunk<D, G, QBF16, true>(p, sm, b, kvh, 0);
    __syncthreads();
    store_final<D, G>(
        p, sm, [&](int w) { return reinterpret_cast<const float*>(&sm.u.stage[w][0][0]); },
        [&](int w) { return reinterpret_cast<const float*>(&sm.u.f8.blk[w][0][0]); }, b, kvh);
    return;
  }
  // One-dimensional grid, dispatched in index order and spread round-robin
  // over the 8 XCDs. The INT8 regions take `pairs` consecutive items, before
  // (int8_first = 1) or after (0) the INT4 chunks; INT4 item j is chunk
  // j / pairs of pair j % pairs (chunk-major: the first, fullest chunks of
  // every sequence go first, and each XCD gets every 8th pair of every chunk
  // index, i.e. the same mix of sequence lengths). Pair = b * Hkv + kvh.
  // Partial index: INT4 chunk j at j, the INT8 region at nsplit.
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
    if constexpr (POOL) {
      int4_pool_chunk<D, G, QBF16, false>(p, sm, b, kvh, split);
      __syncthreads();
      store_partial<D, G, POOL>(sm, [&](int w) { return reinterpret_cast<float*>(&sm.u.stage[w][0][0]); }, dst);
    } else {
      int4_mask_chunk<D, G, QBF16, TIER>(p, sm, b, kvh, split);
      __syncthreads();
      store_partial<D, G, false>(sm, [&](int w) { return &sm.u.w4[w].ro.o[0][0]; }, dst);
    }
  } else {
    // Pool mode, one chunk per pair: the INT8 workgroup usually runs after its
    // chunk has finished (INT8 workgroups are dispatched after the chunks). It
    // reads the pair's count at its start; if the chunk has already counted
    // itself, this workgroup is the last: it loads the chunk's partial while
    // it computes, and merges with its own partial straight from LDS (no
    // partial store, no count), with the merge's exact operations, so the
    // output is the same bits either way.
    const bool peek = POOL && p.nsplit == 1;
    int32_t* ctr = p.pool_header + 4 * (size_t)pair + 3;
    __shared__ int s_fast;
    int seen = -1;
    if (peek && threadIdx.x == 0) seen = __hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    constexpr int kE = (G * D + kThreads - 1) / kThreads;  // output elements per thread
    float c_m[kE], c_l[kE], c_o[kE];
    bool fast = false;
    const float* run = p.parts + ((size_t)b * p.hkv + kvh) * np * G * (2 + D);  // the chunk's partial
    int8_region<D, G, QBF16>(p, sm, b, kvh, [&] {
      if (!peek) return;
      if (threadIdx.x == 0) s_fast = seen == np - 1;
      __syncthreads();
      fast = s_fast != 0;
      if (fast) {
#pragma unroll
        for (int e = 0; e < kE; ++e) {
          const int i = threadIdx.x + kThreads * e;
          const int h = (i < G * D ? i : 0) / D, ch = (i < G * D ? i : 0) % D;
          const float* row = run + (size_t)h * (2 + D);
          c_m[e] = __hip_atomic_load(row, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          c_l[e] = __hip_atomic_load(row + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          c_o[e] = __hip_atomic_load(row + 2 + ch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
    });
    __syncthreads();
    if (POOL && fast) {
#pragma unroll
      for (int e = 0; e < kE; ++e) {
        const int i = threadIdx.x + kThreads * e;
        if (i >= G * D) break;
        const int h = i / D, ch = i % D;
        float M8, o8, l8;
        combine_waves<D, G>(sm, [&](int w) { return &sm.u.i8.o[w][0][0]; }, h, ch, M8, o8, l8);
        // merge_head over the partials (chunk, INT8), operation for operation
        const float M = fmaxf(c_m[e], M8);
        const float w0 = (c_m[e] == -INFINITY || M == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(c_m[e] - M);
        const float w1 = (M8 == -INFINITY || M == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(M8 - M);
        const float den = __builtin_fmaf(w0, c_l[e], 0.0f) + __builtin_fmaf(w1, l8, 0.0f);
        const float acc = __builtin_fmaf(w1, o8, __builtin_fmaf(w0, c_o[e], 0.0f));
        const float inv = den > 0.0f ? 1.0f / den : 0.0f;
        const size_t oq = (size_t)b * p.hkv * G + kvh * G + h;
        p.out[oq * D + ch] = acc * inv;
        if (ch == 0 && p.lse) p.lse[oq] = den > 0.0f ? (M + log2f(den)) * kLn2 : -INFINITY;
      }
      // the count reached np - 1 without this workgroup: it ends at 0
      if (threadIdx.x == 0) __hip_atomic_store(ctr, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return;
    }
    store_partial<D, G, POOL>(sm, [&](int w) { return &sm.u.i8.o[w][0][0]; }, dst);
  }
  if constexpr (POOL) {
    // The last of the pair's np workgroups to finish merges the partials, so
    // no second launch is needed. Word 3 of the pair's header counts finished
    // workgroups: the refresh leaves it 0, and the last workgroup resets it.
    // The partials were stored at device scope (through this XCD's L2) and
    // every wave waits for its stores to complete before the count, so a
    // workgroup that sees the final count reads complete partials with
    // device-scope loads; no L2 writeback or invalidation is needed.
    static_assert(sizeof(sm.u) >= kWaves * kMaxParts * sizeof(float), "merge weights fit the staging area");
    __shared__ int s_last;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0) {
      int32_t* ctr = p.pool_header + 4 * (size_t)pair + 3;
      const int old = __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      s_last = old == np - 1;
      // a count at or past the last (a header the refresh did not write) is
      // cleared too, so the next call starts from 0
      if (old >= np - 1) __hip_atomic_store(ctr, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    if (s_last) {
      const int wave = threadIdx.x >> 6;
      if (wave < G)
        merge_head<D, G, true>(p, b, kvh, wave, threadIdx.x & 63,
                         reinterpret_cast<float*>(&sm.u) + wave * kMaxParts);
    }
  }
}

template <int D, int G>
hipError_t launch_dq(const kvc_cache& c, const AttnParams& p, bool qbf16, bool pool, bool fuse8, hipStream_t s) {
  const dim3 grid((unsigned)(p.nsplit + 1) * c.num_kv_heads * c.batch);
  if (pool && fuse8 && p.nsplit == 1) {  // one workgroup per pair does both regions
    const dim3 g1((unsigned)c.num_kv_heads * c.batch);
    if (qbf16) hipLaunchKernelGGL((attention_kernel<D, G, true, false, true, true>), g1, dim3(kThreads), 0, s, p);
    else hipLaunchKernelGGL((attention_kernel<D, G, false, false, true, true>), g1, dim3(kThreads), 0, s, p);
  } else if (pool) {
    if (qbf16) hipLaunchKernelGGL((attention_kernel<D, G, true, false, true, false>), grid, dim3(kThreads), 0, s, p);
    else hipLaunchKernelGGL((attention_kernel<D, G, false, false, true, false>), grid, dim3(kThreads), 0, s, p);
  } else if (p.host_pages > 0) {
    if (qbf16) hipLaunchKernelGGL((attention_kernel<D, G, true, true, false, false>), grid, dim3(kThreads), 0, s, p);
    else hipLaunchKernelGGL((attention_kernel<D, G, false, true, false, false>), grid, dim3(kThreads), 0, s, p);
  } else {
    if (qbf16) hipLaunchKernelGGL((attention_kernel<D, G, true, false, false, false>), grid, dim3(kThreads), 0, s, p);
    else hipLaunchKernelGGL((attention_kernel<D, G, false, false, false, false>), grid, dim3(kThreads), 0, s, p);
  }
  // pool mode merges inside the attention kernel
  if (!pool) hipLaunchKernelGGL((merge_kernel<D, G>), dim3(G, c.num_kv_heads, c.batch), dim3(64), 0, s, p);
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
  AttnParams p{};
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
  p.errors = c.errors;
  const int G = num_q_heads / c.num_kv_heads;
  if (plan.pool) {
    p.pool = c.pool;
    p.pool_header = c.pool_header;
    p.pool_cap = c.pool_capacity;
  }
  const bool bf = q_dtype == KVC_BF16;
  const bool pool = plan.pool != 0;
  const bool fuse8 = plan.fuse8 != 0;
  if (c.head_dim == 128) {
    switch (G) {
      case 1: return launch_dq<128, 1>(c, p, bf, pool, fuse8, s);
      case 2: return launch_dq<128, 2>(c, p, bf, pool, fuse8, s);
      case 4: return launch_dq<128, 4>(c, p, bf, pool, fuse8, s);
    }
  } else {
    switch (G) {
      case 1: return launch_dq<64, 1>(c, p, bf, pool, fuse8, s);
      case 2: return launch_dq<64, 2>(c, p, bf, pool, fuse8, s);
      case 4: return launch_dq<64, 4>(c, p, bf, pool, fuse8, s);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace kvc
