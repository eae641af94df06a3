// Split-region decode attention over the compressed cache, with the exact
// log-sum-exp merge, in one kernel launch.
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
// (logit * log2 e), l = sum 2^(s - m), o = sum 2^(s - m) * v. A second,
// small kernel merges the nsplit + 1 partials of each (sequence, kv head) in
// index order, so results do not depend on scheduling.
//
// INT4 chunk, per wave (a quarter of the chunk):
//  * The kept positions (keep-mask bits) are compacted with ballot/mbcnt into
//    an LDS list of token-record indices, so evicted tokens cost no HBM reads
//    and every read is a whole token record (K||V codes, 128 B at D = 128).
//    The mask words and block-table entries of the wave's range are fetched
//    with one load each, and the main loop fetches the next 32 tokens while
//    it computes the current ones.
//  * Logits use v_mfma_f32_16x16x32_f16 with the raw codes: a nibble n becomes
//    the fp16 value 1024 + n (or 1024 + 16n) by OR-ing it into 0x6400, which is
//    exact; one MFMA row is one token, one column one (group, head) pair, and
//    the query operand is zero outside the column's own group, so each column
//    accumulates exactly one group's dot product q_g . c_g. The per-group
//    scale and min are then applied in float32:
//      s = sum_g scale_g (q_g . c_g) + min_g sum(q_g)   (rows = tokens).
//  * P.V uses the same MFMA with rows = (group, head) pairs, whose P operand
//    is p * V_scale[token][group] in fp16, and columns = channels 8n + m read
//    from V-code dword n; the codes enter as 1024 + 16c and the 1024 offset
//    plus 16 * 8 (centring the codes) is removed by one extra MFMA against a
//    constant 1152 operand. Only rows whose group matches the column's channel
//    group are kept. The remaining term sum_t p_t (V_min + 8 V_scale)[t][g] is
//    accumulated in float32 on the side.
//  * Softmax: exact running max per head with a wave-uniform rescale branch.
#include "kvc_internal.h"

#include <type_traits>

namespace kvc {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr uint32_t kMagic = 0x64006400u;   // fp16 1024.0 in both halves
constexpr uint32_t kCentre = 0x64806480u;  // fp16 1152.0 = 1024 + 16 * 8 in both halves
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;

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
  int hkv;
  int max_pages;
  int num_pages;
  int max_ctx;
  int words;
  int chunk;
  int nsplit;
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

// LDS shared by the INT4 and INT8 paths of one workgroup.
template <int D, int G>
struct Smem {
  static constexpr int kListCap = 512;  // positions per wave (chunk <= 4 * 512)
  union {
    struct {
      uint64_t code[kWaves][kListCap + 64];  // byte offset of the token's K codes
      uint32_t meta[kWaves][kListCap + 64];  // byte offset of the token's meta row
    } list;
    struct {
      float q[G][D];
      int8_t vcode[kWaves][36][D];
      float vscale[kWaves][36];
      float p[kWaves][G][36];
    } i8;
  } u;
  float o[kWaves][G][D];
  float m[kWaves][G];
  float l[kWaves][G];
  float vm[kWaves][16];
  int32_t pages[kWaves][64];
  uint32_t vbuf[kWaves][32][D / 8];  // V codes of the current 32 tokens
  uint32_t mbuf[kWaves][32][D / 16]; // meta rows of the current 32 tokens
};

// Combine the four waves' (m, l, o) held in LDS into one partial and store it.
template <int D, int G>
__device__ inline void store_partial(const AttnParams& p, Smem<D, G>& sm, float* dst) {
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
        o += a * sm.o[w][h][ch];
        l += a * sm.l[w][h];
      }
    }
    float* row = dst + (size_t)h * (2 + D);
    row[2 + ch] = o;
    if (ch == 0) { row[0] = M; row[1] = l; }
  }
}

// ------------------------------------------------------------------ INT4 chunk
template <int D, int G, bool QBF16>
__device__ void int4_chunk(const AttnParams& p, Smem<D, G>& sm, int b, int kvh, int split) {
  using S = Shape<D, G>;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int s = lane >> 4;          // row slot
  const int n = lane & 15;          // column
  const int gc = (n / G) % S::NG;   // column's group
  const int hc = n % G;             // column's head
  int L = p.seq_lens[b];
  L = L < 0 ? 0 : (L > p.max_ctx ? p.max_ctx : L);
  const int n4 = L > kInt8Slots ? L - kInt8Slots : 0;
  const int r0 = kSink, r1 = kSink + n4;  // INT4 region [r0, r1)
  const int q4 = p.chunk / kWaves;
  const int w0 = split * p.chunk + wave * q4;
  const int lo = w0 > r0 ? w0 : r0;
  const int hi = w0 + q4 < r1 ? w0 + q4 : r1;

  // ---- compact the kept positions of this wave's range into an LDS list
  uint64_t* lcode = sm.u.list.code[wave];
  uint32_t* lmeta = sm.u.list.meta[wave];
  int cnt = 0;
  const uint32_t* mrow = p.mask + ((size_t)b * p.hkv + kvh) * p.words;
  const int32_t* bt = p.block_table + (size_t)b * p.max_pages;
  {
    // one load for the range's mask words (<= 32) and one for its pages (<= 64)
    uint32_t myword = 0;
    int32_t mypage = -1;
    if (lane < q4 / 32 && w0 + 32 * lane < hi) myword = mrow[(w0 >> 5) + lane];
    if (lane < q4 / 16 && w0 + 16 * lane < hi) mypage = bt[(w0 >> 4) + lane];
    sm.pages[wave][lane] = mypage;
    __builtin_amdgcn_wave_barrier();
    for (int r = 0; w0 + 64 * r < hi; ++r) {
      const uint32_t wlo = __builtin_amdgcn_readlane(myword, 2 * r);
      const uint32_t whi = __builtin_amdgcn_readlane(myword, 2 * r + 1);
      const uint64_t bits = (uint64_t)wlo | ((uint64_t)whi << 32);
      const int pos = w0 + 64 * r + lane;
      const int page = sm.pages[wave][(64 * r + lane) >> 4];
      const bool kept = ((bits >> lane) & 1u) && pos >= lo && pos < hi && page >= 0 &&
                        page < p.num_pages;
      const uint64_t bal = __ballot(kept);
      if (kept) {
        const int rank = __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32),
                                                   __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0));
        const uint32_t rec = ((uint32_t)page * p.hkv + kvh) * kPage + (pos & (kPage - 1));
        lcode[cnt + rank] = (uint64_t)rec * D;
        lmeta[cnt + rank] = rec * (uint32_t)(S::NG * 8);
      }
      cnt += __popcll(bal);
    }
  }
  if (cnt > 0) {
    // pad to a whole tile plus one more, so the prefetch never needs a branch
    const uint64_t fc = lcode[0];
    const uint32_t fm = lmeta[0];
    const int padded = ((cnt + 31) & ~31) + 32;
    if (cnt + lane < padded) { lcode[cnt + lane] = fc; lmeta[cnt + lane] = fm; }
  }

  float m_col = -INFINITY, l_col = 0.0f, vm_col = 0.0f;
  float4v acc[8], acc_off = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int m = 0; m < 8; ++m) acc[m] = acc_off;

  if (cnt > 0) {
    // ---- query operands: column (gc, hc) holds q for group gc only
    const int hq = kvh * G + hc;
    const size_t qoff = ((size_t)b * p.hkv * G + hq) * D;
    const int slot_group = (s * D / 4) / 32;
    const bool active = slot_group == gc;
    half8 bq[S::NG];
    float off = 0.0f, qsum = 0.0f;
    const int perm[8] = {0, 4, 1, 5, 2, 6, 3, 7};
#pragma unroll
    for (int m = 0; m < S::NG; ++m) {
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const int code = s * (D / 4) + 8 * m + perm[r];
        const bool x16 = (r == 2 || r == 3 || r == 6 || r == 7);
        float qv = load_q<QBF16>(p.q, qoff + code);
        qv = active ? qv : 0.0f;
        qsum += qv;
        const _Float16 qh = (_Float16)(x16 ? qv * 0.0625f : qv);
        bq[m][r] = qh;
        off += (float)qh * 1024.0f;
      }
    }
    // every code of the column's group sits in exactly one active slot
    qsum = rows_sum(qsum);
    // the column's offset sums over all four k-slots (rows of the B operand)
    off = rows_sum(off);
    const float alpha = p.alpha;
    const float a_off = alpha * off;
    const float a_qs = alpha * qsum;

    // ---- main loop over 32 kept tokens per iteration, next tokens prefetched
    // A tile in flight: K codes in MFMA operand order (token n and 16 + n,
    // slot s), and for token lane/2 one half of its V codes and of its meta row.
    struct Tile {
      uint32_t kd0[S::NG], kd1[S::NG];
      uint32_t vh[S::VD / 2];
      uint32_t mh[S::NG];
    };
    const int vdw = n % S::VD;
    const int tl = lane >> 1, hf = lane & 1;
    const uint8_t* kbase = p.codes + s * S::SB;
    const uint8_t* vbase = p.codes + D / 2 + hf * (D / 4);
    const uint8_t* mbase = reinterpret_cast<const uint8_t*>(p.meta) + hf * (D / 8);
    uint32_t* vrow = sm.vbuf[wave][tl] + hf * (S::VD / 2);
    uint32_t* mrow_l = sm.mbuf[wave][tl] + hf * (S::NG);
    auto fetch = [&](int it, Tile& t) {
      const uint64_t o0 = lcode[it + n], o1 = lcode[it + 16 + n];
      const uint64_t ov = lcode[it + tl];
      const uint32_t om = lmeta[it + tl];
      if constexpr (D == 128) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(kbase + o0);
        const u32x4 c = *reinterpret_cast<const u32x4*>(kbase + o1);
        const u32x4 v0 = *reinterpret_cast<const u32x4*>(vbase + ov);
        const u32x4 v1 = *reinterpret_cast<const u32x4*>(vbase + ov + 16);
        const u32x4 mm = *reinterpret_cast<const u32x4*>(mbase + om);
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          t.kd0[m] = a[m]; t.kd1[m] = c[m]; t.vh[m] = v0[m]; t.vh[4 + m] = v1[m]; t.mh[m] = mm[m];
        }
      } else {
        const u32x2 a = *reinterpret_cast<const u32x2*>(kbase + o0);
        const u32x2 c = *reinterpret_cast<const u32x2*>(kbase + o1);
        const u32x4 v0 = *reinterpret_cast<const u32x4*>(vbase + ov);
        const u32x2 mm = *reinterpret_cast<const u32x2*>(mbase + om);
#pragma unroll
        for (int m = 0; m < 2; ++m) { t.kd0[m] = a[m]; t.kd1[m] = c[m]; t.mh[m] = mm[m]; }
#pragma unroll
        for (int m = 0; m < 4; ++m) t.vh[m] = v0[m];
      }
    };
    auto compute = [&](const Tile& cur, int it, auto tail) {
      const uint32_t* kd0 = cur.kd0;
      const uint32_t* kd1 = cur.kd1;
#pragma unroll
      for (int m = 0; m < S::VD / 2; ++m) vrow[m] = cur.vh[m];
#pragma unroll
      for (int m = 0; m < S::NG; ++m) mrow_l[m] = cur.mh[m];
      __builtin_amdgcn_wave_barrier();
      uint32_t vd[8];
      u32x2 md[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int tok = i < 4 ? 4 * s + i : 16 + 4 * s + (i - 4);
        vd[i] = sm.vbuf[wave][tok][vdw];
        md[i] = *reinterpret_cast<const u32x2*>(&sm.mbuf[wave][tok][2 * gc]);
      }

      // QK: C[token][(g,h)] = q_g . c_g
      float4v c0 = {0.0f, 0.0f, 0.0f, 0.0f}, c1 = c0;
#pragma unroll
      for (int m = 0; m < S::NG; ++m) {
        uint32_t x = kd0[m];
        uint32_t y = x >> 8;
        half8 a = as_half8(and_or(x, 0x000F000Fu, kMagic), and_or(x, 0x00F000F0u, kMagic),
                           and_or(y, 0x000F000Fu, kMagic), and_or(y, 0x00F000F0u, kMagic));
        c0 = mfma16x16x32(a, bq[m], c0);
        x = kd1[m];
        y = x >> 8;
        a = as_half8(and_or(x, 0x000F000Fu, kMagic), and_or(x, 0x00F000F0u, kMagic),
                     and_or(y, 0x000F000Fu, kMagic), and_or(y, 0x00F000F0u, kMagic));
        c1 = mfma16x16x32(a, bq[m], c1);
      }
      float sv[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float d = i < 4 ? c0[i] : c1[i - 4];
        const float ks = h2f(md[i][0] & 0xFFFFu), km = h2f(md[i][0] >> 16);
        const float e = fmaf(d, alpha, -a_off);
        sv[i] = fmaf(ks, e, km * a_qs);
      }
      // sum the group columns of each head (columns h, h+G, h+2G, ... within a row)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if constexpr (S::NC >= 2 * G) sv[i] += row_ror<G>(sv[i]);
        if constexpr (S::NC >= 4 * G) sv[i] += row_ror<2 * G>(sv[i]);
        if constexpr (S::NC >= 8 * G) sv[i] += row_ror<4 * G>(sv[i]);
        if constexpr (S::NC >= 16 * G) sv[i] += row_ror<8 * G>(sv[i]);
      }
      if constexpr (decltype(tail)::value) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int tok = i < 4 ? 4 * s + i : 16 + 4 * s + (i - 4);
          if (it + tok >= cnt) sv[i] = -INFINITY;
        }
      }
      // running max per head, rescale only when it grows
      float bm = sv[0];
#pragma unroll
      for (int i = 1; i < 8; ++i) bm = fmaxf(bm, sv[i]);
      bm = rows_max(bm);
      if (__ballot(bm > m_col)) {
        const float mn = fmaxf(m_col, bm);
        const float a = mn == -INFINITY ? 1.0f : __builtin_amdgcn_exp2f(m_col - mn);
        m_col = mn;
        l_col *= a;
        vm_col *= a;
        float ah[G];
#pragma unroll
        for (int h = 0; h < G; ++h)
          ah[h] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, a), h));
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float f = ah[j % G];
#pragma unroll
          for (int m = 0; m < 8; ++m) acc[m][j] *= f;
          acc_off[j] *= f;
        }
      }
      float pp[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float pr = __builtin_amdgcn_exp2f(sv[i] - m_col);
        l_col += pr;
        const float vsc = h2f(md[i][1] & 0xFFFFu);
        vm_col = fmaf(pr, fmaf(8.0f, vsc, h2f(md[i][1] >> 16)), vm_col);
        pp[i] = pr * vsc;
      }
      const half8 A = as_half8(pack_f16x2(pp[0], pp[1]), pack_f16x2(pp[2], pp[3]),
                               pack_f16x2(pp[4], pp[5]), pack_f16x2(pp[6], pp[7]));
      // P.V: V codes of tokens (2q, 2q+1) paired into fp16 halves 1024 + 16c
      uint32_t xlo[4], xhi[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        xlo[q] = __builtin_amdgcn_perm(vd[2 * q + 1], vd[2 * q], 0x05040100u);
        xhi[q] = __builtin_amdgcn_perm(vd[2 * q + 1], vd[2 * q], 0x07060302u);
      }
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        uint32_t bw[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t x = m < 4 ? xlo[q] : xhi[q];
          const int mm = m & 3;
          const uint32_t y = mm == 0 ? (x << 4) : mm == 1 ? x : mm == 2 ? (x >> 4) : (x >> 8);
          bw[q] = and_or(y, 0x00F000F0u, kMagic);
        }
        acc[m] = mfma16x16x32(A, as_half8(bw[0], bw[1], bw[2], bw[3]), acc[m]);
      }
      acc_off = mfma16x16x32(A, as_half8(kCentre, kCentre, kCentre, kCentre), acc_off);
      __builtin_amdgcn_wave_barrier();
    };
    // whole tiles ping-pong between two register sets; the last tile (which
    // may hold padding) masks its invalid tokens
    using Full = std::integral_constant<bool, false>;
    using Tail = std::integral_constant<bool, true>;
    const int last = (cnt - 1) & ~31;
    Tile t0, t1;
    fetch(0, t0);
    int it = 0;
    for (;;) {
      fetch(it + 32, t1);
      if (it == last) { compute(t0, it, Tail{}); break; }
      compute(t0, it, Full{});
      it += 32;
      fetch(it + 32, t0);
      if (it == last) { compute(t1, it, Tail{}); break; }
      compute(t1, it, Full{});
      it += 32;
    }
    l_col = rows_sum(l_col);
    vm_col = rows_sum(vm_col);
  }

  // ---- this wave's (m, l, o) into LDS
  if (lane < G) {
    sm.m[wave][lane] = m_col;  // lane h < G has column (0, h)
    sm.l[wave][lane] = l_col;
  }
  if (lane < 16) sm.vm[wave][lane] = vm_col;
  __builtin_amdgcn_s_waitcnt(0);
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int row = 4 * s + j;
    const int g = (row / G) % S::NG, h = row % G;
    const bool ok = row < S::NC && g == n / 4 && n < S::VD && cnt > 0;
    if (ok) {
      const float vmin = sm.vm[wave][g * G + h];
#pragma unroll
      for (int m = 0; m < 8; ++m)
        sm.o[wave][h][8 * n + m] = (acc[m][j] - acc_off[j]) * 0.0625f + vmin;
    }
  }
  if (cnt == 0) {
    for (int i = lane; i < G * D; i += 64) sm.o[wave][i / D][i % D] = 0.0f;
  }
}

// ------------------------------------------------------------------ INT8 region
// The <= 144 protected positions of one (sequence, kv head) in float32: each
// wave takes 36 positions, lane = token for the logits, lane = channels for P.V.
template <int D, int G, bool QBF16>
__device__ void int8_region(const AttnParams& p, Smem<D, G>& sm, int b, int kvh) {
  constexpr int CPL = D / 64;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  int L = p.seq_lens[b];
  L = L < 0 ? 0 : (L > p.max_ctx ? p.max_ctx : L);
  const int ns = L < kSink ? L : kSink;
  const int rr0 = L - kRecent > kSink ? L - kRecent : kSink;
  const int nr = L > rr0 ? L - rr0 : 0;
  const int n8 = ns + nr;
  for (int i = threadIdx.x; i < G * D; i += kThreads) {
    const int h = i / D, d = i % D;
    sm.u.i8.q[h][d] = load_q<QBF16>(p.q, ((size_t)b * p.hkv * G + kvh * G + h) * D + d) * p.alpha;
  }
  __syncthreads();
  const int i0 = wave * 36;
  const int cntw = n8 - i0 < 0 ? 0 : (n8 - i0 > 36 ? 36 : n8 - i0);
  const size_t base = ((size_t)b * p.hkv + kvh) * kInt8Slots;
  float s[G];
#pragma unroll
  for (int h = 0; h < G; ++h) s[h] = -INFINITY;
  const bool valid = lane < cntw;
  if (valid) {
    const int idx = i0 + lane;
    const int pos = idx < ns ? idx : rr0 + (idx - ns);
    const int slot = pos < kSink ? pos : kSink + (pos - kSink) % kRecent;
    const int8_t* kc = p.codes8 + (base + slot) * 2 * D;
    const float ks = p.scales8[(base + slot) * 2 + 0];
    const float vs = p.scales8[(base + slot) * 2 + 1];
    float dot[G];
#pragma unroll
    for (int h = 0; h < G; ++h) dot[h] = 0.0f;
    for (int d0 = 0; d0 < D; d0 += 16) {
      const u32x4 w4 = *reinterpret_cast<const u32x4*>(kc + d0);
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const float c = (float)(int8_t)(w4[k / 4] >> (8 * (k % 4)));
#pragma unroll
        for (int h = 0; h < G; ++h) dot[h] = fmaf(sm.u.i8.q[h][d0 + k], c, dot[h]);
      }
    }
#pragma unroll
    for (int h = 0; h < G; ++h) s[h] = ks * dot[h];
    for (int d0 = 0; d0 < D; d0 += 16)
      *reinterpret_cast<u32x4*>(&sm.u.i8.vcode[wave][lane][d0]) = *reinterpret_cast<const u32x4*>(kc + D + d0);
    sm.u.i8.vscale[wave][lane] = vs;
  }
  float m[G], l[G], o[G][CPL];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float mx = s[h];
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
    m[h] = mx;
    const float pr = valid ? __builtin_amdgcn_exp2f(s[h] - mx) : 0.0f;
    float sum = pr;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) sum += __shfl_xor(sum, off);
    l[h] = sum;
    if (lane < 36) sm.u.i8.p[wave][h][lane] = pr * (valid ? sm.u.i8.vscale[wave][lane] : 0.0f);
#pragma unroll
    for (int c = 0; c < CPL; ++c) o[h][c] = 0.0f;
  }
  __builtin_amdgcn_s_waitcnt(0);
  __builtin_amdgcn_wave_barrier();
  for (int j = 0; j < cntw; ++j) {
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const float v = (float)sm.u.i8.vcode[wave][j][lane * CPL + c];
#pragma unroll
      for (int h = 0; h < G; ++h) o[h][c] = fmaf(sm.u.i8.p[wave][h][j], v, o[h][c]);
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
    for (int c = 0; c < CPL; ++c) sm.o[wave][h][lane * CPL + c] = o[h][c];
}

// ------------------------------------------------------------------ merge
// One workgroup per (query head, kv head, sequence) merges the nsplit + 1
// partials in index order: M = max_j m_j, w_j = 2^(m_j - M) (0 for empty
// partials), out = sum_j w_j o_j / sum_j w_j l_j,
// lse = ln 2 * (M + log2 sum_j w_j l_j). All loads are issued in parallel:
// one (m, l) pair per thread, then D/4 float4 columns x 8 partial sums.
template <int D, int G>
__global__ __launch_bounds__(kThreads) void merge_kernel(AttnParams p) {
  constexpr int kMaxParts = 256;  // the host plan keeps nsplit + 1 <= 256
  constexpr int NF = D / 4;       // float4 columns
  constexpr int R = kThreads / NF;  // threads per column
  __shared__ float wts[kMaxParts];
  __shared__ float red[kThreads / 64][2];
  __shared__ float4v part_acc[kThreads];
  const int h = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int np = p.nsplit + 1;
  const float* parts = p.parts + ((size_t)b * p.hkv + kvh) * np * G * (2 + D) + (size_t)h * (2 + D);
  const size_t pstride = (size_t)G * (2 + D);
  float mj = -INFINITY, lj = 0.0f;
  if (tid < np) {
    const float2v ml = *reinterpret_cast<const float2v*>(parts + tid * pstride);
    mj = ml[0];
    lj = ml[1];
  }
  float M = mj;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
  if (lane == 0) red[wid][0] = M;
  __syncthreads();
  M = red[0][0];
#pragma unroll
  for (int w = 1; w < kThreads / 64; ++w) M = fmaxf(M, red[w][0]);
  const float wj = (mj == -INFINITY || M == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(mj - M);
  if (tid < np) wts[tid] = wj;
  float den = wj * lj;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) den += __shfl_xor(den, o);
  __syncthreads();
  if (lane == 0) red[wid][1] = den;
  __syncthreads();
  den = 0.0f;
#pragma unroll
  for (int w = 0; w < kThreads / 64; ++w) den += red[w][1];
  const int c4 = tid % NF, r = tid / NF;
  float4v acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll 8
  for (int j = r; j < np; j += R) {
    const float w = wts[j];
    if (w != 0.0f) acc += w * *reinterpret_cast<const float4v*>(parts + j * pstride + 2 + 4 * c4);
  }
  part_acc[tid] = acc;
  __syncthreads();
  if (r == 0) {
#pragma unroll
    for (int q = 1; q < R; ++q) acc += part_acc[q * NF + c4];
    const float inv = den > 0.0f ? 1.0f / den : 0.0f;
    const size_t oq = (size_t)b * p.hkv * G + kvh * G + h;
    *reinterpret_cast<float4v*>(p.out + oq * D + 4 * c4) = acc * inv;
    if (c4 == 0 && p.lse) p.lse[oq] = den > 0.0f ? (M + log2f(den)) * kLn2 : -INFINITY;
  }
}

template <int D, int G, bool QBF16>
__global__ __launch_bounds__(kThreads) void attention_kernel(AttnParams p) {
  __shared__ Smem<D, G> sm;
  // blockIdx.x: split (nsplit = INT8 region), blockIdx.y: kv head, blockIdx.z: sequence
  const int split = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  if (split < p.nsplit) int4_chunk<D, G, QBF16>(p, sm, b, kvh, split);
  else int8_region<D, G, QBF16>(p, sm, b, kvh);
  __syncthreads();
  const int np = p.nsplit + 1;
  float* dst = p.parts + (((size_t)b * p.hkv + kvh) * np + split) * G * (2 + D);
  store_partial<D, G>(p, sm, dst);
}

template <int D, int G>
hipError_t launch_dq(const kvc_cache& c, const AttnParams& p, bool qbf16, hipStream_t s) {
  const dim3 grid(p.nsplit + 1, c.num_kv_heads, c.batch);
  if (qbf16) hipLaunchKernelGGL((attention_kernel<D, G, true>), grid, dim3(kThreads), 0, s, p);
  else hipLaunchKernelGGL((attention_kernel<D, G, false>), grid, dim3(kThreads), 0, s, p);
  hipLaunchKernelGGL((merge_kernel<D, G>), dim3(G, c.num_kv_heads, c.batch), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attention(const kvc_cache& c, const void* q, kvc_dtype q_dtype, int num_q_heads,
                            float softmax_scale, float* out, float* lse, float* ws,
                            const AttnPlan& plan, hipStream_t s) {
  AttnParams p;
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
  p.max_pages = c.max_pages_per_seq;
  p.num_pages = c.num_phys_pages;
  p.max_ctx = c.max_ctx;
  p.words = mask_words(c.max_ctx);
  p.chunk = plan.chunk;
  p.nsplit = plan.nsplit;
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
