// Dense bfloat16 paged-KV decode attention: the uncompressed baseline.
//
// Source: KV4-RL review, section 3 - the INT4 cache's rollout speedups are
// measured against BF16 rollout, whose KV cache holds every K and V row in
// bfloat16 and whose decode attention reads every cached position. This file
// is that baseline on the same paging, split-KV decomposition and exact
// log-sum-exp merge as the compressed path, so the two compare call for call.
//
// Layout: kv (bfloat16 bits) [P][Hkv][16][2][D] - per token the K row then the
// V row, 4D bytes (512 B at D = 128); block_table and seq_lens as in the
// compressed cache.
//
// Work: one workgroup (4 waves) per (sequence, kv head, chunk of positions);
// each wave walks a quarter of the chunk in 32-token tiles (two pages), with
// the next tile's loads in flight during the current tile's arithmetic:
//  * Logits: v_mfma_f32_16x16x32_bf16 with rows = 16 tokens, taken straight
//    from the K rows as loaded (lane l holds 8 channels of token l % 16), and
//    columns = query heads. The scaled query enters as two bfloat16 parts,
//    hi = rne(q) in column h and lo = rne(q - hi) in column G + h; their sum
//    carries ~16 significant bits and the products are exact, so the logits
//    are float32-accurate (s = C[h] + C[G + h], in log2 units).
//  * Softmax: a running max per head, refreshed only when a tile's max
//    exceeds it by more than 8 (log2 units), so p = 2^(s - m) < 2^8; p goes
//    to LDS, one row of G values per token.
//  * P.V in float32 on the vector ALUs: lane = (token, 8 channels) of each V
//    load, reading its token's p row; every lane owns fixed channels, and the
//    lanes sharing channels are summed once at the end.
// The workgroup's four waves are combined into one partial (m, l, o) per
// query head (m in log2 units), merged across chunks by the merge kernel of
// the compressed path.
#include "kvc_internal.h"

namespace kvc {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kTile = 32;  // tokens per wave step (two pages)

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

struct DenseParams {
  const uint16_t* kv;
  const int32_t* block_table;
  const int32_t* seq_lens;
  const void* q;
  float* parts;  // [B][Hkv][nsplit][G][2 + D]
  float alpha;   // softmax scale * log2(e)
  int batch, hkv, max_pages, num_pages, max_ctx, chunk, nsplit;
};

__device__ inline float4v mfma_bf16(u32x4 a, u32x4 b, float4v c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// bfloat16 bits of x, round to nearest even (NaN -> quiet NaN)
__device__ inline uint32_t bf16_rne(float x) {
  const uint32_t u = __float_as_uint(x);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x40u;
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ inline float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// lane i of each 16-lane row takes v from lane i + N of its row (0 past the row's end)
template <int N>
__device__ inline float row_shl(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x100 + N, 0xF, 0xF, true));
}

// eight consecutive query values from element off (a multiple of 8)
template <bool QBF16>
__device__ inline void load_q8(const void* q, size_t off, float (&x)[8]) {
  if constexpr (QBF16) {
    const u32x4 w = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(q) + off);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      x[2 * k] = bf16_lo(w[k]);
      x[2 * k + 1] = bf16_hi(w[k]);
    }
  } else {
    const float4v* f = reinterpret_cast<const float4v*>(reinterpret_cast<const float*>(q) + off);
    const float4v a = f[0], c = f[1];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      x[k] = a[k];
      x[4 + k] = c[k];
    }
  }
}

template <int D, int G>
struct DenseSmem {
  float p[kWaves][kTile][G];  // the current tile's p, one row of G heads per token
  float corr[kWaves][4];      // factors of the current max refresh, per head
  float m[kWaves][G];
  float l[kWaves][G];
  float o[kWaves][G][D];
};

template <int D, int G, bool QBF16>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) void dense_attention_kernel(
    DenseParams p) {
  constexpr int KS = D / 32;        // MFMA k-steps per 16 tokens
  constexpr int LPR = D / 8;        // lanes per V row (16 B each)
  constexpr int TPI = 64 / LPR;     // tokens per V load (4 or 8)
  constexpr int NVI = kTile / TPI;  // V loads per tile
  constexpr int RS = 2 * D;         // elements per token record
  static_assert(2 * G <= 16, "hi and lo query columns fit one MFMA tile");
  __shared__ DenseSmem<D, G> sm;
  // One-dimensional grid, chunk-major: item j is chunk j / pairs of pair j % pairs.
  const int pairs = p.hkv * p.batch;
  const int pair = blockIdx.x % pairs, split = blockIdx.x / pairs;
  const int kvh = pair % p.hkv, b = pair / p.hkv;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 15, row = lane >> 4;
  int L = p.seq_lens[b];
  L = L < 0 ? 0 : (L > p.max_ctx ? p.max_ctx : L);
  const int span = p.chunk / kWaves;  // positions per wave (multiple of 32)
  const int w0 = split * p.chunk + wave * span;
  const int w1 = w0 + span < L ? w0 + span : L;

  // query operand: column c holds head c (hi part) or head c - G (lo part), zero beyond 2G
  u32x4 qb[KS];
  {
    const bool used = col < 2 * G;
    const int h = col < G ? col : (used ? col - G : 0);
    const size_t qoff = ((size_t)b * p.hkv * G + (size_t)kvh * G + h) * D + 8 * row;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      float x[8];
      load_q8<QBF16>(p.q, qoff + 32 * s, x);
      uint32_t hv[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float y = used ? x[i] * p.alpha : 0.0f;
        const uint32_t hi = bf16_rne(y);
        hv[i] = col < G ? hi : bf16_rne(y - __uint_as_float(hi << 16));
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) qb[s][i] = hv[2 * i] | (hv[2 * i + 1] << 16);
    }
  }
  // physical page ids of the wave's range (up to 128 pages), -1 where invalid
  int pg[2];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int lp = w0 / kPage + lane + 64 * r;
    int id = -1;
    if (lp < p.max_pages && lp * kPage < w1) {
      id = p.block_table[(size_t)b * p.max_pages + lp];
      if (id < 0 || id >= p.num_pages) id = -1;
    }
    pg[r] = id;
  }

  float m = -INFINITY, lsum = 0.0f;  // head `col` (lanes with col < G)
  float o[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int k = 0; k < 8; ++k) o[h][k] = 0.0f;

  struct TileRegs {
    u32x4 k[2][KS];
    u32x4 v[NVI];
    int ok;  // bit g: page g of the tile is valid
  };
  auto page_of = [&](int t0, int g) -> int {
    const int i = (t0 - w0) / kPage + g;  // wave-uniform
    return __builtin_amdgcn_readlane(i < 64 ? pg[0] : pg[1], i & 63);
  };
  auto load_tile = [&](int t0, TileRegs& r) {
    const uint16_t* base[2];
    r.ok = 0;
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      const int id = page_of(t0, g);
      r.ok |= (id >= 0) << g;
      base[g] = p.kv + ((size_t)(id >= 0 ? id : 0) * p.hkv + kvh) * (kPage * RS);
    }
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int s = 0; s < KS; ++s)
        r.k[g][s] = *reinterpret_cast<const u32x4*>(base[g] + col * RS + 32 * s + 8 * row);
#pragma unroll
    for (int i = 0; i < NVI; ++i) {
      const int tt = i * TPI + lane / LPR;
      r.v[i] = *reinterpret_cast<const u32x4*>(base[tt / kPage] + (tt % kPage) * RS + D +
                                                8 * (lane % LPR));
    }
  };
  auto compute_tile = [&](int t0, const TileRegs& r) {
    // logits of the tile's 32 tokens: lane (row, col) holds tokens 16g + 4 row + j for column col
    float s[2][4];
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      float4v c = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) c = mfma_bf16(r.k[g][ks], qb[ks], c);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int pos = t0 + 16 * g + 4 * row + j;
        const float x = c[j] + row_shl<G>(c[j]);
        s[g][j] = (pos < L && ((r.ok >> g) & 1)) ? x : -INFINITY;
      }
    }
    float tm = fmaxf(fmaxf(fmaxf(s[0][0], s[0][1]), fmaxf(s[0][2], s[0][3])),
                     fmaxf(fmaxf(s[1][0], s[1][1]), fmaxf(s[1][2], s[1][3])));
    tm = fmaxf(tm, __shfl_xor(tm, 16));
    tm = fmaxf(tm, __shfl_xor(tm, 32));
    // lazy refresh of the running max (heads whose tile max passed m + 8)
    const bool need = col < G && tm > m + 8.0f;
    if (__ballot(need)) {
      const float mn = need ? fmaxf(m, tm) : m;
      const float cf = need ? __builtin_amdgcn_exp2f(m - mn) : 1.0f;  // m = -inf gives 0
      lsum *= cf;
      m = mn;
      if (lane < G) sm.corr[wave][lane] = cf;
      // a wave's LDS operations complete in order: the reads below see the write
      __builtin_amdgcn_wave_barrier();
      float cr[G];
#pragma unroll
      for (int h = 0; h < G; ++h) cr[h] = sm.corr[wave][h];
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int k = 0; k < 8; ++k) o[h][k] *= cr[h];
    }
    if (col < G) {
#pragma unroll
      for (int g = 0; g < 2; ++g)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float x = s[g][j];
          const float pv = x == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(x - m);
          lsum += pv;
          sm.p[wave][16 * g + 4 * row + j][col] = pv;
        }
    }
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int i = 0; i < NVI; ++i) {
      const int tt = i * TPI + lane / LPR;
      float pr[G];
#pragma unroll
      for (int h = 0; h < G; ++h) pr[h] = sm.p[wave][tt][h];
      float v[8];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        v[2 * k] = bf16_lo(r.v[i][k]);
        v[2 * k + 1] = bf16_hi(r.v[i][k]);
      }
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int k = 0; k < 8; ++k) o[h][k] = fmaf(pr[h], v[k], o[h][k]);
    }
    __builtin_amdgcn_wave_barrier();
  };

  // two register sets, alternating: the next tile loads while this one
  // computes. The loads are unconditional, so that each compute waits only for
  // its own set; past the last tile they repeat the last tile (cache hits).
  if (w0 < w1) {
    const int last = w0 + (w1 - w0 - 1) / kTile * kTile;
    TileRegs ra, rb;
    load_tile(w0, ra);
    for (int t0 = w0;;) {
      load_tile(t0 + kTile <= last ? t0 + kTile : last, rb);
      compute_tile(t0, ra);
      t0 += kTile;
      if (t0 > last) break;
      load_tile(t0 + kTile <= last ? t0 + kTile : last, ra);
      compute_tile(t0, rb);
      t0 += kTile;
      if (t0 > last) break;
    }
  }

  // lanes sharing channels (same lane % LPR) hold disjoint tokens: sum them
#pragma unroll
  for (int x = LPR; x < 64; x <<= 1)
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int k = 0; k < 8; ++k) o[h][k] += __shfl_xor(o[h][k], x);
  lsum += __shfl_xor(lsum, 16);
  lsum += __shfl_xor(lsum, 32);
  if (lane < G) {
    sm.m[wave][lane] = m;
    sm.l[wave][lane] = lsum;
  }
  if (lane < LPR) {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int k = 0; k < 8; ++k) sm.o[wave][h][8 * lane + k] = o[h][k];
  }
  __syncthreads();
  // combine the four waves into this chunk's partial
  float* dst = p.parts + (((size_t)b * p.hkv + kvh) * p.nsplit + split) * G * (2 + D);
  for (int i = threadIdx.x; i < G * D; i += kThreads) {
    const int h = i / D, ch = i % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sm.m[w][h]);
    float acc = 0.0f, l = 0.0f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float mw = sm.m[w][h];
        if (mw == -INFINITY) continue;
        const float a = __builtin_amdgcn_exp2f(mw - M);
        acc += a * sm.o[w][h][ch];
        l += a * sm.l[w][h];
      }
    }
    float* rowp = dst + (size_t)h * (2 + D);
    rowp[2 + ch] = acc;
    if (ch == 0) {
      rowp[0] = M;
      rowp[1] = l;
    }
  }
}

// ------------------------------------------------------------------ append
// One thread per 8 elements of one K or V row of one appended token.
struct DenseAppendParams {
  uint16_t* kv;
  const int32_t* block_table;
  const int32_t* seq_lens;
  const void* k_new;
  const void* v_new;
  const int32_t* n_new;
  int batch, hkv, n_new_max, max_pages, num_pages, max_ctx;
  long long items;
};

template <int D, bool BF16>
__global__ __launch_bounds__(256) void dense_append_kernel(DenseAppendParams p) {
  const long long it = (long long)blockIdx.x * 256 + threadIdx.x;
  if (it >= p.items) return;
  constexpr int E = D / 8;
  const int e = (int)(it % E);
  long long r = it / E;
  const int which = (int)(r % 2);
  r /= 2;
  const int h = (int)(r % p.hkv);
  r /= p.hkv;
  const int j = (int)(r % p.n_new_max);
  const int b = (int)(r / p.n_new_max);
  const int n = p.n_new[b];
  if (j >= n) return;
  const int t = p.seq_lens[b] - n + j;
  if (t < 0 || t >= p.max_ctx) return;
  const int id = p.block_table[(size_t)b * p.max_pages + t / kPage];
  if (id < 0 || id >= p.num_pages) return;
  const size_t src = (((size_t)b * p.n_new_max + j) * p.hkv + h) * D + 8 * e;
  const void* base = which ? p.v_new : p.k_new;
  u32x4 w;
  if constexpr (BF16) {
    w = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(base) + src);
  } else {
    const float4v* f = reinterpret_cast<const float4v*>(reinterpret_cast<const float*>(base) + src);
    const float4v a = f[0], c = f[1];
    w[0] = bf16_rne(a[0]) | (bf16_rne(a[1]) << 16);
    w[1] = bf16_rne(a[2]) | (bf16_rne(a[3]) << 16);
    w[2] = bf16_rne(c[0]) | (bf16_rne(c[1]) << 16);
    w[3] = bf16_rne(c[2]) | (bf16_rne(c[3]) << 16);
  }
  uint16_t* dst = p.kv + (((size_t)id * p.hkv + h) * kPage + t % kPage) * (2 * D) + which * D + 8 * e;
  *reinterpret_cast<u32x4*>(dst) = w;
}

template <int D>
hipError_t launch_dense_attention_d(const DenseParams& p, int G, bool qbf16, hipStream_t s) {
  const dim3 grid((unsigned)p.nsplit * p.hkv * p.batch), block(kThreads);
  switch (G) {
    case 1:
      if (qbf16) hipLaunchKernelGGL((dense_attention_kernel<D, 1, true>), grid, block, 0, s, p);
      else hipLaunchKernelGGL((dense_attention_kernel<D, 1, false>), grid, block, 0, s, p);
      break;
    case 2:
      if (qbf16) hipLaunchKernelGGL((dense_attention_kernel<D, 2, true>), grid, block, 0, s, p);
      else hipLaunchKernelGGL((dense_attention_kernel<D, 2, false>), grid, block, 0, s, p);
      break;
    case 4:
      if (qbf16) hipLaunchKernelGGL((dense_attention_kernel<D, 4, true>), grid, block, 0, s, p);
      else hipLaunchKernelGGL((dense_attention_kernel<D, 4, false>), grid, block, 0, s, p);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_dense_append(const kvc_dense_cache& c, const void* k_new, const void* v_new,
                               kvc_dtype src, int n_new_max, const int32_t* n_new, hipStream_t s) {
  DenseAppendParams p;
  p.kv = c.kv;
  p.block_table = c.block_table;
  p.seq_lens = c.seq_lens;
  p.k_new = k_new;
  p.v_new = v_new;
  p.n_new = n_new;
  p.batch = c.batch;
  p.hkv = c.num_kv_heads;
  p.n_new_max = n_new_max;
  p.max_pages = c.max_pages_per_seq;
  p.num_pages = c.num_phys_pages;
  p.max_ctx = c.max_ctx;
  p.items = (long long)c.batch * n_new_max * c.num_kv_heads * 2 * (c.head_dim / 8);
  const dim3 grid((unsigned)((p.items + 255) / 256)), block(256);
  const bool bf = src == KVC_BF16;
  if (c.head_dim == 128) {
    if (bf) hipLaunchKernelGGL((dense_append_kernel<128, true>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((dense_append_kernel<128, false>), grid, block, 0, s, p);
  } else {
    if (bf) hipLaunchKernelGGL((dense_append_kernel<64, true>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((dense_append_kernel<64, false>), grid, block, 0, s, p);
  }
  return hipGetLastError();
}

hipError_t launch_dense_attention(const kvc_dense_cache& c, const void* q, kvc_dtype q_dtype,
                                  int num_q_heads, float softmax_scale, float* out, float* lse,
                                  float* ws, const DensePlan& plan, hipStream_t s) {
  DenseParams p;
  p.kv = c.kv;
  p.block_table = c.block_table;
  p.seq_lens = c.seq_lens;
  p.q = q;
  p.parts = ws;
  p.alpha = softmax_scale * kLog2e;
  p.batch = c.batch;
  p.hkv = c.num_kv_heads;
  p.max_pages = c.max_pages_per_seq;
  p.num_pages = c.num_phys_pages;
  p.max_ctx = c.max_ctx;
  p.chunk = plan.chunk;
  p.nsplit = plan.nsplit;
  const int G = num_q_heads / c.num_kv_heads;
  const bool bf = q_dtype == KVC_BF16;
  hipError_t e = c.head_dim == 128 ? launch_dense_attention_d<128>(p, G, bf, s)
                                   : launch_dense_attention_d<64>(p, G, bf, s);
  if (e != hipSuccess) return e;
  return launch_merge(ws, plan.nsplit, c.batch, c.num_kv_heads, G, c.head_dim, out, lse, s);
}

}  // namespace kvc
