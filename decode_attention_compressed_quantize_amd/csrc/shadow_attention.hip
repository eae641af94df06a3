// Learner-side causal attention under the recorded shadow mask (Shadow Mask
// Distillation page, section 1 and Figure 1 caption: the keep mask of every
// rollout step is injected into the learner's causal attention, so that each
// generated position's query attends to exactly what the rollout attended).
//
// One workgroup per (sequence, kv head, tile of R query rows); R = 32 * 8 / G,
// so that each wave owns 32 rows (two MFMA row blocks sharing every K and V
// operand read) of one query head and the waves share every key tile. Per span
// of up to 2048 / (R / 32) key positions the workgroup lists the keys that
// any of its rows attends (prompt rows: all keys up to the row; generated rows:
// the shadow row's bits up to the row) together with an R-bit mask of which
// rows attend each one, then walks the list 32 keys at a time:
//   - K and V rows of the 32 keys into LDS (gathers of 16-byte pieces; the
//     listed positions are arbitrary);
//   - S^T = K Q^T with bf16 MFMA 16x16x32 (Q operands held in registers), so
//     that each lane holds eight keys of one query row;
//   - masked online softmax in log2 units, lane-local: the row maximum is
//     refreshed (across the row's four lanes) only when a score passes it by a
//     fixed slack, and row sums are reduced once at the end;
//   - O^T += V^T P^T with bf16 MFMA, V^T through transposing LDS reads, P^T
//     straight from registers, split into a high and a low bf16 part so that
//     P keeps ~16 significant bits.
// Nothing is computed for keys no row of the tile attends.

#include "kvc_internal.h"

namespace kvc {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kSaThreads = 512;
constexpr int kSaWaves = 8;
constexpr int kStep = 32;   // listed keys per MFMA step
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct ShadowParams {
  const uint16_t* q;  // bf16 [B][max_len][Hq][D]
  const uint16_t* k;  // bf16 [B][max_len][Hkv][D]
  const uint16_t* v;
  const int32_t* seq_lens;
  const int32_t* prompt_lens;
  const uint32_t* shadow;  // [B][Hkv][rows][words]
  float* out;              // [B][max_len][Hq][D]
  float* lse;              // [B][max_len][Hq] or null
  int batch, max_len, hq, hkv, words, rows, tiles;
  float alpha;  // softmax scale * log2(e)
};

template <int D, int G>
struct SaSmem {
  static constexpr int R = 32 * (kSaWaves / G);  // query rows per workgroup (32 per wave)
  static constexpr int NRW = R / 32;             // 32-row words of a key's row mask
  static constexpr int SPAN = 2048 / NRW;        // key positions listed at a time
  // Row strides (bf16 elements) that keep the 16-byte operand reads free of
  // bank conflicts: LDS serves them 32 lanes at a time over 128 four-byte
  // banks, so the 32 lanes' 16-byte pieces (16 rows x 2 column chunks) must
  // fall on distinct bank quadruples.
  static constexpr int KS = D + 16;  // K and V rows: 72 or 40 dwords apart
  alignas(16) uint16_t k[2][kStep][KS];  // two buffers each: a step computes from one
  alignas(16) uint16_t v[2][kStep][KS];  // while later keys are written into the other
  alignas(16) uint32_t rmask[NRW][SPAN];  // listed key x: bit i of word q = row r0 + 32q + i attends it
  uint32_t rw[R][SPAN / 32];     // the tile rows' attended-key words over the span
  uint32_t pos[SPAN];            // listed key positions
  uint32_t wcnt[kSaWaves];
};

__device__ inline float4v mfma_bf16(u32x4 a, u32x4 b, float4v c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// S^T = K Q^T leaves lane group g (lanes 16g .. 16g + 15) with keys 4g .. 4g + 3
// and 16 + 4g .. 16 + 4g + 3 of its query row; taking those eight keys as MFMA
// k indices 8g .. 8g + 7 makes the lane's probabilities the B operand of
// O^T = V^T P^T as they stand. The V^T operand in that key order comes from V
// rows in LDS through two transposing reads (ds_read_b64_tr_b16): within a
// 16-lane group, lane 4m + q addresses head_dim entries d0 + 4q .. + 3 of key m
// and lane i receives entry d0 + i of keys 0 .. 3.
typedef short short4v __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) short4v lds_short4v;
__device__ inline uint2 read_tr16(const uint16_t* p) {
  const short4v r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4v*)(p));
  return __builtin_bit_cast(uint2, r);
}

// Piece x (0 .. 32 * D / 8 - 1) of a 32-key step: key and head_dim chunk. The
// 32 lanes of a half wave take 16 keys x 2 chunks, so their 16-byte K writes
// fall on distinct bank quadruples.
__device__ inline int piece_key(int x) { return (x & 15) | (((x >> 5) & 1) << 4); }
__device__ inline int piece_chunk(int x) { return ((x >> 4) & 1) | ((x >> 6) << 1); }

// s where bit i of w is set, else -inf
__device__ inline float keep_or_neg_inf(float s, uint32_t w, int i) {
  const uint32_t keep = (uint32_t)__builtin_amdgcn_sbfe((int)w, i, 1);
  return __uint_as_float((__float_as_uint(s) & keep) | (0xFF800000u & ~keep));
}

// Scores may exceed the row maximum used for the exponentials by this much
// (log2 units) before the maximum is refreshed: probabilities stay below 2^8.
constexpr float kSlack = 8.0f;

template <int D, int G>
__global__ __launch_bounds__(kSaThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void shadow_attention_kernel(ShadowParams p) {
  using S = SaSmem<D, G>;
  constexpr int R = S::R, NRW = S::NRW;
  constexpr int NC = D / 32;  // MFMA k-chunks over head_dim
  constexpr int NT = D / 16;  // output head_dim tiles
  constexpr int kPieces = kStep * (D / 8);  // 16-byte K (and V) pieces per step
  constexpr int NL = (kPieces + kSaThreads - 1) / kSaThreads;  // per thread
  __shared__ S sm;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int pairs = p.hkv * p.batch;
  const int tile = p.tiles - 1 - (int)blockIdx.x / pairs;  // the longest rows first
  const int pair = (int)blockIdx.x % pairs;
  const int h = pair % p.hkv, b = pair / p.hkv;
  int L = p.seq_lens[b];
  L = L < 0 ? 0 : (L > p.max_len ? p.max_len : L);
  int P = p.prompt_lens[b];
  P = P < 0 ? 0 : (P > L ? L : P);
  const int r0 = tile * R;
  if (r0 >= L) return;
  const int rend = r0 + R < L ? r0 + R : L;  // rows [r0, rend), keys [0, rend)
  const int g = wave % G, rb = wave / G;
  const int qh = h * G + g;
  const int wrow0 = r0 + 32 * rb;  // this wave's 32 rows: two MFMA column blocks of 16
  const int lg = lane >> 4;        // lane group: keys 4lg .. 4lg + 3 of each 16-key tile

  // Q operands (B of S^T = K Q^T): lane holds row wrow0 + 16 * blk + lane % 16,
  // head_dim entries 32c + 8 * (lane / 16) .. + 7 of chunk c
  u32x4 qa[2][NC];
#pragma unroll
  for (int blk = 0; blk < 2; ++blk) {
    const int row = wrow0 + 16 * blk + (lane & 15);
    const uint16_t* qp = p.q + (((size_t)b * p.max_len + row) * p.hq + qh) * D + 8 * lg;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const u32x4 zero = {0u, 0u, 0u, 0u};
      qa[blk][c] = row < L ? *reinterpret_cast<const u32x4*>(qp + 32 * c) : zero;
    }
  }

  // Per lane and column block: the query row wrow0 + 16 * blk + lane % 16. m is
  // the row maximum the exponentials are taken against (log2 units, the same in
  // the row's four lane groups), lsum the lane's share of the row sum, o the
  // O^T tiles (head_dim 16t + 4 * (lane / 16) + j of the row).
  float m[2], nm[2], cap[2], lsum[2];
  float4v o[2][NT];
#pragma unroll
  for (int blk = 0; blk < 2; ++blk) {
    m[blk] = -INFINITY;
    nm[blk] = 0.0f;
    cap[blk] = -INFINITY;  // raw scores above cap refresh the maximum
    lsum[blk] = 0.0f;
#pragma unroll
    for (int t = 0; t < NT; ++t) o[blk][t] = float4v{0.0f, 0.0f, 0.0f, 0.0f};
  }
  const float inv_alpha = 1.0f / p.alpha;

  const uint32_t* srow = p.shadow + ((size_t)b * p.hkv + h) * p.rows * (size_t)p.words;
  const uint64_t below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
  for (int cb = 0; cb < rend; cb += S::SPAN) {
    const int ce = cb + S::SPAN < rend ? cb + S::SPAN : rend;
    const int nw = (ce - cb + 31) / 32;
    // ---- the rows' attended-key words over the span (causal limit applied)
    for (int x = threadIdx.x; x < R * nw; x += kSaThreads) {
      const int i = x / nw, w = x % nw;
      const int row = r0 + i;
      const int j0 = cb + 32 * w;
      uint32_t bits = 0;
      if (row < rend) {
        if (row < P) {
          bits = ~0u;
        } else {
          const int r = row - P;
          bits = r < p.rows ? srow[(size_t)r * p.words + (j0 >> 5)] : 0u;
        }
        const int lim = row - j0 + 1;  // keys j0 .. row are causal
        bits &= lim >= 32 ? ~0u : (lim <= 0 ? 0u : ((1u << lim) - 1u));
      }
      sm.rw[i][w] = bits;
    }
    __syncthreads();
    // ---- list the keys any row attends, in position order, with their row masks
    int total = 0;
    for (int kb = 0; kb < ce - cb; kb += kSaThreads) {
      const int jl = kb + (int)threadIdx.x;
      uint32_t rm[NRW];
      bool keep = false;
#pragma unroll
      for (int q = 0; q < NRW; ++q) rm[q] = 0;
      if (cb + jl < ce) {
        const int w = jl >> 5, bit = jl & 31;
#pragma unroll
        for (int q = 0; q < NRW; ++q) {
#pragma unroll 8
          for (int i = 0; i < 32; ++i) rm[q] |= ((sm.rw[32 * q + i][w] >> bit) & 1u) << i;
          keep = keep || rm[q] != 0;
        }
      }
      const uint64_t bal = __ballot(keep);
      if (lane == 0) sm.wcnt[wave] = (uint32_t)__popcll(bal);
      __syncthreads();
      int base = total, add = 0;
#pragma unroll
      for (int q = 0; q < kSaWaves; ++q) {
        const int c = (int)sm.wcnt[q];
        if (q < wave) base += c;
        add += c;
      }
      if (keep) {
        const int at = base + (int)__popcll(bal & below);
        sm.pos[at] = (uint32_t)(cb + jl);
#pragma unroll
        for (int q = 0; q < NRW; ++q) sm.rmask[q][at] = rm[q];
      }
      total += add;
      __syncthreads();
    }
    // pad to whole steps with attended-by-none copies of the first listed key
    const int padded = (total + kStep - 1) / kStep * kStep;
    for (int x = total + (int)threadIdx.x; x < padded; x += kSaThreads) {
      sm.pos[x] = sm.pos[0];
#pragma unroll
      for (int q = 0; q < NRW; ++q) sm.rmask[q][x] = 0;
    }
    __syncthreads();

    // ---- 32 listed keys per step, software-pipelined: while step s's
    // probabilities are formed (VALU), the MFMA unit computes step s + 1's
    // scores, so K runs one step ahead of V. LDS holds K(s + 1) and V(s)
    // during step s, which writes K(s + 2) and V(s + 1) (gathered into
    // registers during step s - 1) into the buffers read in step s - 1 and
    // gathers K(s + 3) and V(s + 2). Thread piece x covers one key and one
    // 8-element head_dim chunk (see piece_key / piece_chunk). Step indices past
    // the end are clamped to the last step: their loads stay in bounds and
    // their results are never used.
    const int nsteps = padded / kStep;
    typedef u32x4 Pieces[NL];
    auto gather = [&](const uint16_t* src, int st, Pieces& r) {
      st = st < nsteps ? st : nsteps - 1;
#pragma unroll
      for (int u = 0; u < NL; ++u) {
        const int x = (int)threadIdx.x + u * kSaThreads;
        if (kPieces % kSaThreads != 0 && x >= kPieces) continue;
        const int e = piece_key(x), c = piece_chunk(x);
        r[u] = *reinterpret_cast<const u32x4*>(
            src + (((size_t)b * p.max_len + sm.pos[st * kStep + e]) * p.hkv + h) * D + 8 * c);
      }
    };
    auto stage = [&](uint16_t (&dst)[kStep][S::KS], const Pieces& r) {
#pragma unroll
      for (int u = 0; u < NL; ++u) {
        const int x = (int)threadIdx.x + u * kSaThreads;
        if (kPieces % kSaThreads != 0 && x >= kPieces) continue;
        *reinterpret_cast<u32x4*>(&dst[piece_key(x)][8 * piece_chunk(x)]) = r[u];
      }
    };
    // S^T = K Q^T from K buffer kb: tile t2 holds keys 16 t2 .. + 15 (rows) of
    // the block's 16 query rows (columns); chunk-outer order keeps four
    // independent accumulators between dependent MFMAs
    auto scores = [&](int kb, float4v (&st)[2][2]) {
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2) st[blk][t2] = float4v{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int c = 0; c < NC; ++c) {
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2) {
          const u32x4 ka = *reinterpret_cast<const u32x4*>(&sm.k[kb][16 * t2 + (lane & 15)][32 * c + 8 * lg]);
          st[0][t2] = mfma_bf16(ka, qa[0][c], st[0][t2]);
          st[1][t2] = mfma_bf16(ka, qa[1][c], st[1][t2]);
        }
      }
    };
    float4v st[2][2];
    Pieces ka_, va_, kb_, vb_;  // two register sets that swap roles every step
    if (nsteps > 0) {
      gather(p.k, 0, ka_);
      gather(p.v, 0, va_);
      gather(p.k, 1, kb_);
      stage(sm.k[0], ka_);
      stage(sm.v[0], va_);
      stage(sm.k[1], kb_);
      gather(p.k, 2, ka_);
      gather(p.v, 1, va_);
      __syncthreads();
      scores(0, st);
      __syncthreads();  // step 0 overwrites K(0) with K(2)
    }
    // kst / vst hold K(s + 2) / V(s + 1); kld / vld receive K(s + 3) / V(s + 2)
    auto step = [&](int s, const Pieces& kst, const Pieces& vst, Pieces& kld, Pieces& vld) {
      const int s0 = s * kStep;
      gather(p.k, s + 3, kld);
      gather(p.v, s + 2, vld);
      // row masks of the lane's eight keys; skipped when the wave's 32 rows attend all 32 keys
      const u32x4 wa = *reinterpret_cast<const u32x4*>(&sm.rmask[rb][s0 + 4 * lg]);
      const u32x4 wb = *reinterpret_cast<const u32x4*>(&sm.rmask[rb][s0 + 16 + 4 * lg]);
      const uint32_t every = wa[0] & wa[1] & wa[2] & wa[3] & wb[0] & wb[1] & wb[2] & wb[3];
      if (__ballot(every != ~0u) != 0) {
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) {
          const int i = 16 * blk + (lane & 15);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            st[blk][0][j] = keep_or_neg_inf(st[blk][0][j], wa[j], i);
            st[blk][1][j] = keep_or_neg_inf(st[blk][1][j], wb[j], i);
          }
        }
      }
      // refresh a block's row maxima only where some score passed its cap
      bool up[2];
      float lmax[2];
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) {
        const float4v x = st[blk][0], y = st[blk][1];
        lmax[blk] = fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])), fmaxf(fmaxf(y[0], y[1]), fmaxf(y[2], y[3])));
        up[blk] = lmax[blk] > cap[blk];
      }
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) {
        if (__ballot(up[blk]) == 0) continue;
        float mx = lmax[blk];
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float mn = fmaxf(m[blk], mx * p.alpha);
        const float ms = mn == -INFINITY ? 0.0f : mn;
        const float corr = __builtin_amdgcn_exp2f(m[blk] - ms);
        m[blk] = mn;
        nm[blk] = -ms;
        cap[blk] = (mn + kSlack) * inv_alpha;
        lsum[blk] *= corr;
#pragma unroll
        for (int t = 0; t < NT; ++t) o[blk][t] *= corr;
      }
      // next step's scores: independent of the exponentials below, so the
      // scheduler can overlap the two
      float4v sn[2][2];
      u32x4 va[NT];
      scores((s + 1) & 1, sn);
      // P^T = exp2(alpha S^T - m): high + low bf16 parts (round to nearest even,
      // hardware conversion), already in the B operand layout of O^T = V^T P^T
      u32x4 ph[2], pl[2];
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) {
        float pv[8];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          pv[j] = __builtin_amdgcn_exp2f(__builtin_fmaf(st[blk][0][j], p.alpha, nm[blk]));
          pv[4 + j] = __builtin_amdgcn_exp2f(__builtin_fmaf(st[blk][1][j], p.alpha, nm[blk]));
        }
        lsum[blk] += ((pv[0] + pv[1]) + (pv[2] + pv[3])) + ((pv[4] + pv[5]) + (pv[6] + pv[7]));
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bf16x2 hi = {(__bf16)pv[2 * e], (__bf16)pv[2 * e + 1]};
          const uint32_t hw = __builtin_bit_cast(uint32_t, hi);
          const float h0 = __uint_as_float(hw << 16), h1 = __uint_as_float(hw & 0xFFFF0000u);
          const bf16x2 lo = {(__bf16)(pv[2 * e] - h0), (__bf16)(pv[2 * e + 1] - h1)};
          ph[blk][e] = hw;
          pl[blk][e] = __builtin_bit_cast(uint32_t, lo);
        }
      }
      // O^T += V^T P^T (A = V^T head_dim rows x keys, B = P^T keys x query rows):
      // every V^T operand read once, high parts first so that the two MFMAs
      // into one accumulator sit 2 * NT apart
      {
        const uint16_t* vb = &sm.v[s & 1][4 * lg + ((lane & 15) >> 2)][4 * (lane & 3)];
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const uint2 a = read_tr16(vb + 16 * t), c = read_tr16(vb + 16 * S::KS + 16 * t);
          va[t] = u32x4{a.x, a.y, c.x, c.y};
        }
      }
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) o[blk][t] = mfma_bf16(va[t], ph[blk], o[blk][t]);
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) o[blk][t] = mfma_bf16(va[t], pl[blk], o[blk][t]);
      stage(sm.k[s & 1], kst);
      stage(sm.v[(s + 1) & 1], vst);
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2) st[blk][t2] = sn[blk][t2];
      __syncthreads();
    };
    for (int s = 0; s < nsteps; s += 2) {
      step(s, ka_, va_, kb_, vb_);
      if (s + 1 < nsteps) step(s + 1, kb_, vb_, ka_, va_);
    }
  }

  // ---- out = O / l, lse = ln 2 * (m + log2 l); rows that attend nothing get 0 and -inf
#pragma unroll
  for (int blk = 0; blk < 2; ++blk) {
    float l = lsum[blk];
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    const int row = wrow0 + 16 * blk + (lane & 15);
    if (row >= L) continue;
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
    float* op = p.out + (((size_t)b * p.max_len + row) * p.hq + qh) * D + 4 * lg;
#pragma unroll
    for (int t = 0; t < NT; ++t) *reinterpret_cast<float4v*>(op + 16 * t) = o[blk][t] * inv;
    if (p.lse && lg == 0)
      p.lse[((size_t)b * p.max_len + row) * p.hq + qh] = l > 0.0f ? (m[blk] + log2f(l)) * kLn2 : -INFINITY;
  }
}

template <int D, int G>
void launch_dg(const ShadowParams& p, hipStream_t s) {
  hipLaunchKernelGGL((shadow_attention_kernel<D, G>), dim3((unsigned)(p.tiles * p.hkv * p.batch)),
                     dim3(kSaThreads), 0, s, p);
}

}  // namespace

hipError_t launch_shadow_attention(const void* q, const void* k, const void* v, int batch,
                                   int max_len, int num_q_heads, int num_kv_heads, int head_dim,
                                   const int32_t* seq_lens, const int32_t* prompt_lens,
                                   const uint32_t* shadow, int shadow_rows, float softmax_scale,
                                   float* out, float* lse, hipStream_t s) {
  ShadowParams p;
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.seq_lens = seq_lens;
  p.prompt_lens = prompt_lens;
  p.shadow = shadow;
  p.out = out;
  p.lse = lse;
  p.batch = batch;
  p.max_len = max_len;
  p.hq = num_q_heads;
  p.hkv = num_kv_heads;
  p.words = (max_len + 31) / 32;
  p.rows = shadow_rows;
  p.alpha = softmax_scale * kLog2e;
  const int G = num_q_heads / num_kv_heads;
  const int R = 32 * (kSaWaves / G);
  p.tiles = (max_len + R - 1) / R;
  if (head_dim == 128) {
    if (G == 4) launch_dg<128, 4>(p, s);
    else if (G == 2) launch_dg<128, 2>(p, s);
    else launch_dg<128, 1>(p, s);
  } else {
    if (G == 4) launch_dg<64, 4>(p, s);
    else if (G == 2) launch_dg<64, 2>(p, s);
    else launch_dg<64, 1>(p, s);
  }
  return hipGetLastError();
}

}  // namespace kvc
