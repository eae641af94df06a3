// Learner-side causal attention under the recorded shadow mask (Shadow Mask
// Distillation page, section 1 and Figure 1 caption: the keep mask of every
// rollout step is injected into the learner's causal attention, so that each
// generated position's query attends to exactly what the rollout attended).
//
// One workgroup per (sequence, kv head, tile of R query rows); R = 32 * 4 / G,
// so that each wave owns 32 rows (two MFMA row blocks sharing every K and V
// operand read) of one query head and the waves share every key tile. Per span
// of 512 key positions the workgroup lists the keys that
// any of its rows attends (prompt rows: all keys up to the row; generated rows:
// the shadow row's bits up to the row) together with an R-bit mask of which
// rows attend each one, then walks the list 32 keys at a time:
//   - K rows of the 32 keys into LDS, V rows transposed into LDS (gathers of
//     16-byte pieces; the listed positions are arbitrary);
//   - S = Q K^T with bf16 MFMA 16x16x32 (Q operands held in registers);
//   - masked online softmax in log2 units (row reductions over a 16-lane DPP row);
//   - O += P V with bf16 MFMA, P split into a high and a low bf16 part so that
//     P keeps ~16 significant bits.
// Nothing is computed for keys no row of the tile attends.

#include "kvc_internal.h"

namespace kvc {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kSaThreads = 256;
constexpr int kSaWaves = 4;
constexpr int kStep = 32;   // listed keys per MFMA step
constexpr int kSpan = 512;  // key positions listed at a time
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
  static constexpr int KS = D + 8;               // K row stride (bf16 elements)
  static constexpr int VS = kStep + 8;           // V^T row stride
  static constexpr int PS = kStep + 8;           // P row stride
  alignas(16) uint16_t k[2][kStep][KS];  // two buffers: step s computes from one while
  alignas(16) uint16_t vt[2][D][VS];     // step s + 1's keys are written into the other
  alignas(16) uint16_t ph[kSaWaves][2][16][PS];
  alignas(16) uint16_t pl[kSaWaves][2][16][PS];
  uint32_t rw[R][kSpan / 32];     // the tile rows' attended-key words over the span
  uint32_t pos[kSpan];            // listed key positions
  uint32_t rmask[kSpan][NRW];     // per listed key: bit i of word q = row r0 + 32q + i attends it
  uint32_t wcnt[kSaWaves];
};

__device__ inline float4v mfma_bf16(u32x4 a, u32x4 b, float4v c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Max and sum over the 16 lanes of a DPP row (one row of the MFMA C layout):
// swap neighbours, swap pairs, mirror within 8, mirror within 16. Every lane
// ends with the row's result.
template <int Ctrl>
__device__ inline float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), Ctrl, 0xF, 0xF, false));
}
__device__ inline float row16_max(float x) {
  x = fmaxf(x, dpp<0xB1>(x));   // quad_perm [1,0,3,2]
  x = fmaxf(x, dpp<0x4E>(x));   // quad_perm [2,3,0,1]
  x = fmaxf(x, dpp<0x141>(x));  // row_half_mirror
  return fmaxf(x, dpp<0x140>(x));  // row_mirror
}
__device__ inline float row16_sum(float x) {
  x += dpp<0xB1>(x);
  x += dpp<0x4E>(x);
  x += dpp<0x141>(x);
  return x + dpp<0x140>(x);
}


template <int D, int G>
__global__ __launch_bounds__(kSaThreads) void shadow_attention_kernel(ShadowParams p) {
  using S = SaSmem<D, G>;
  constexpr int R = S::R, NRW = S::NRW;
  constexpr int NC = D / 32;  // MFMA k-chunks over head_dim
  constexpr int NT = D / 16;  // output column tiles
  constexpr int NL = kStep * (D / 8) / kSaThreads;  // 16-byte K (and V) pieces per thread per step
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
  const int wrow0 = r0 + 32 * rb;  // this wave's 32 rows: two MFMA row blocks of 16

  // Q operands (A of QK^T): lane holds row wrow0 + 16 * blk + lane % 16,
  // head_dim entries 32c + 8 * (lane / 16) .. + 7 of chunk c
  u32x4 qa[2][NC];
#pragma unroll
  for (int blk = 0; blk < 2; ++blk) {
    const int row = wrow0 + 16 * blk + (lane & 15);
    const uint16_t* qp = p.q + (((size_t)b * p.max_len + row) * p.hq + qh) * D + 8 * (lane >> 4);
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const u32x4 zero = {0u, 0u, 0u, 0u};
      qa[blk][c] = row < L ? *reinterpret_cast<const u32x4*>(qp + 32 * c) : zero;
    }
  }

  // lane's rows in the C layout: 16 * blk + 4 * (lane / 16) + jj of the wave's 32
  const int lr = 4 * (lane >> 4);
  float m[2][4], l[2][4];
  float4v o[2][NT];
#pragma unroll
  for (int blk = 0; blk < 2; ++blk) {
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      m[blk][jj] = -INFINITY;
      l[blk][jj] = 0.0f;
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) o[blk][t] = float4v{0.0f, 0.0f, 0.0f, 0.0f};
  }

  const uint32_t* srow = p.shadow + ((size_t)b * p.hkv + h) * p.rows * (size_t)p.words;
  const uint64_t below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
  for (int cb = 0; cb < rend; cb += kSpan) {
    const int ce = cb + kSpan < rend ? cb + kSpan : rend;
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
        for (int q = 0; q < NRW; ++q) sm.rmask[at][q] = rm[q];
      }
      total += add;
      __syncthreads();
    }
    // pad to whole steps with attended-by-none copies of the first listed key
    const int padded = (total + kStep - 1) / kStep * kStep;
    for (int x = total + (int)threadIdx.x; x < padded; x += kSaThreads) {
      sm.pos[x] = sm.pos[0];
#pragma unroll
      for (int q = 0; q < NRW; ++q) sm.rmask[x][q] = 0;
    }
    __syncthreads();

    // ---- 32 listed keys per step. Thread piece x covers key x % 32 and
    // head_dim chunk x / 32 (so a wave's V^T writes fill consecutive banks);
    // the next step's pieces are loaded while this one computes.
    u32x4 kr[NL], vr[NL];
    auto gather = [&](int s0) {
#pragma unroll
      for (int u = 0; u < NL; ++u) {
        const int x = (int)threadIdx.x + u * kSaThreads;
        const int e = x % kStep, c = x / kStep;
        const size_t off = (((size_t)b * p.max_len + sm.pos[s0 + e]) * p.hkv + h) * D + 8 * c;
        kr[u] = *reinterpret_cast<const u32x4*>(p.k + off);
        vr[u] = *reinterpret_cast<const u32x4*>(p.v + off);
      }
    };
    auto stage = [&](int buf) {
#pragma unroll
      for (int u = 0; u < NL; ++u) {
        const int x = (int)threadIdx.x + u * kSaThreads;
        const int e = x % kStep, c = x / kStep;
        *reinterpret_cast<u32x4*>(&sm.k[buf][e][8 * c]) = kr[u];
#pragma unroll
        for (int t = 0; t < 8; ++t) sm.vt[buf][8 * c + t][e] = (uint16_t)(vr[u][t >> 1] >> (16 * (t & 1)));
      }
    };
    if (padded > 0) {
      gather(0);
      stage(0);
    }
    __syncthreads();
    for (int s0 = 0, buf = 0; s0 < padded; s0 += kStep, buf ^= 1) {
      const bool more = s0 + kStep < padded;
      if (more) gather(s0 + kStep);
      // S = Q K^T for both row blocks; each K operand read once
      float4v sacc[2][2];
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2) sacc[blk][t2] = float4v{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2) {
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          const u32x4 kb4 =
              *reinterpret_cast<const u32x4*>(&sm.k[buf][16 * t2 + (lane & 15)][32 * c + 8 * (lane >> 4)]);
          sacc[0][t2] = mfma_bf16(qa[0][c], kb4, sacc[0][t2]);
          sacc[1][t2] = mfma_bf16(qa[1][c], kb4, sacc[1][t2]);
        }
      }
      const uint32_t rmA = sm.rmask[s0 + (lane & 15)][rb];
      const uint32_t rmB = sm.rmask[s0 + 16 + (lane & 15)][rb];
      float corr[2][4];
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) {
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int i = 16 * blk + lr + jj;
          const float sa = ((rmA >> i) & 1u) ? sacc[blk][0][jj] * p.alpha : -INFINITY;
          const float sb = ((rmB >> i) & 1u) ? sacc[blk][1][jj] * p.alpha : -INFINITY;
          const float mx = row16_max(fmaxf(sa, sb));
          const float mn = fmaxf(m[blk][jj], mx);
          const float ms = mn == -INFINITY ? 0.0f : mn;
          corr[blk][jj] = __builtin_amdgcn_exp2f(m[blk][jj] - ms);
          const float pa = __builtin_amdgcn_exp2f(sa - ms);
          const float pb = __builtin_amdgcn_exp2f(sb - ms);
          const float rs = row16_sum(pa + pb);
          l[blk][jj] = l[blk][jj] * corr[blk][jj] + rs;
          m[blk][jj] = mn;
          // P = high + low bf16 parts (round to nearest even, hardware conversion)
          const int pr = lr + jj;
          const bf16x2 hi = {(__bf16)pa, (__bf16)pb};
          const bf16x2 lo = {(__bf16)(pa - (float)hi[0]), (__bf16)(pb - (float)hi[1])};
          const uint32_t hw = __builtin_bit_cast(uint32_t, hi), lw = __builtin_bit_cast(uint32_t, lo);
          sm.ph[wave][blk][pr][lane & 15] = (uint16_t)hw;
          sm.ph[wave][blk][pr][16 + (lane & 15)] = (uint16_t)(hw >> 16);
          sm.pl[wave][blk][pr][lane & 15] = (uint16_t)lw;
          sm.pl[wave][blk][pr][16 + (lane & 15)] = (uint16_t)(lw >> 16);
        }
        // O needs rescaling only where a row maximum rose (corr < 1)
        const bool rose = corr[blk][0] != 1.0f || corr[blk][1] != 1.0f || corr[blk][2] != 1.0f ||
                          corr[blk][3] != 1.0f;
        if (__ballot(rose) != 0) {
#pragma unroll
          for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) o[blk][t][jj] *= corr[blk][jj];
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      // O += P V (A = P rows x keys, B = V^T keys x head_dim columns), each V operand read once
      u32x4 pha[2], pla[2];
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) {
        pha[blk] = *reinterpret_cast<const u32x4*>(&sm.ph[wave][blk][lane & 15][8 * (lane >> 4)]);
        pla[blk] = *reinterpret_cast<const u32x4*>(&sm.pl[wave][blk][lane & 15][8 * (lane >> 4)]);
      }
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const u32x4 vb = *reinterpret_cast<const u32x4*>(&sm.vt[buf][16 * t + (lane & 15)][8 * (lane >> 4)]);
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) {
          o[blk][t] = mfma_bf16(pha[blk], vb, o[blk][t]);
          o[blk][t] = mfma_bf16(pla[blk], vb, o[blk][t]);
        }
      }
      if (more) stage(buf ^ 1);  // the other buffer was last read in the previous step
      __syncthreads();
    }
  }

  // ---- out = O / l, lse = ln 2 * (m + log2 l); rows that attend nothing get 0 and -inf
#pragma unroll
  for (int blk = 0; blk < 2; ++blk) {
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int row = wrow0 + 16 * blk + lr + jj;
      if (row >= L) continue;
      const float inv = l[blk][jj] > 0.0f ? 1.0f / l[blk][jj] : 0.0f;
      float* op = p.out + (((size_t)b * p.max_len + row) * p.hq + qh) * D + (lane & 15);
#pragma unroll
      for (int t = 0; t < NT; ++t) op[16 * t] = o[blk][t][jj] * inv;
      if (p.lse && (lane & 15) == 0)
        p.lse[((size_t)b * p.max_len + row) * p.hq + qh] =
            l[blk][jj] > 0.0f ? (m[blk][jj] + log2f(l[blk][jj])) * kLn2 : -INFINITY;
    }
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
