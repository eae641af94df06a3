// Per-head scoring MLP and budgeted top-k keep mask (the shadow mask).
//
// Sources: KVP promo page (arXiv 2602.10238), section "Core mechanism" - one
// small MLP per attention head reads the K/V vectors and emits a utility
// score per token; deployment is score -> sort -> truncate to the budget.
// Shadow Mask Distillation page (arXiv 2605.06850), Figure 1 caption - the
// eviction records the retained indices in a binary mask.
//
// Scoring: one wave per (kv head, run of tokens). Lane (u, half) holds row u
// of W1 restricted to K (half 0) or V (half 1) in registers, so W1 is read
// once per wave; each token's K||V is staged in LDS as float32 and every lane
// takes a broadcast dot product, then the two halves and the 32 hidden units
// are combined with shuffles.
//
// Top-k: one workgroup per (sequence, kv head). An exact radix select over
// order-preserving 32-bit keys (4 passes of 8 bits, MSB first) finds the
// k-th key T and how many keys equal to T must be kept; a final in-order pass
// keeps every key > T and the lowest-position keys == T, which is the unique
// answer under "score descending, then position ascending". Scores are
// static once written, so refreshing from scratch equals any incremental
// update.
#include "kvc_internal.h"

namespace kvc {
namespace {

// ----------------------------------------------------------------- scoring
struct ScoreParams {
  const float* mlp;
  const void* k_new;
  const void* v_new;
  const int32_t* n_new;
  const int32_t* seq_lens;
  float* scores;
  int batch;
  int hkv;
  int n_new_max;
  int max_ctx;
  int tokens_per_wave;
  int waves_per_head;
};

template <int D, bool BF16>
__global__ __launch_bounds__(64) void score_kernel(ScoreParams p) {
  __shared__ float xs[2 * D];
  const int lane = threadIdx.x;
  const int h = blockIdx.x / p.waves_per_head;
  const int w = blockIdx.x % p.waves_per_head;
  const int u = lane & 31;
  const int half = lane >> 5;
  const float* wh = p.mlp + (size_t)h * mlp_floats(D);
  float w1[D];
#pragma unroll
  for (int i = 0; i < D; i += 4) {
    const float4 f = *reinterpret_cast<const float4*>(wh + (size_t)u * 2 * D + half * D + i);
    w1[i] = f.x; w1[i + 1] = f.y; w1[i + 2] = f.z; w1[i + 3] = f.w;
  }
  const float b1 = wh[kHidden * 2 * D + u];
  const float w2 = wh[kHidden * 2 * D + kHidden + u];
  const float b2 = wh[kHidden * 2 * D + 2 * kHidden];

  const long long total = (long long)p.batch * p.n_new_max;
  const long long f0 = (long long)w * p.tokens_per_wave;
  const long long f1 = f0 + p.tokens_per_wave < total ? f0 + p.tokens_per_wave : total;
  for (long long f = f0; f < f1; ++f) {
    const int b = (int)(f / p.n_new_max);
    const int j = (int)(f % p.n_new_max);
    const int nn = p.n_new[b];
    if (j >= nn) continue;
    const int L = p.seq_lens[b];
    const int pos = L - nn + j;
    if (pos < 0 || pos >= p.max_ctx) continue;
    const size_t src = (((size_t)b * p.n_new_max + j) * p.hkv + h) * D;
    __syncthreads();
    // stage K||V as float32: 2D values, 2D/64 per lane
#pragma unroll
    for (int i = lane; i < 2 * D; i += 64) {
      const int which = i / D;
      const int d = i % D;
      const void* base = which ? p.v_new : p.k_new;
      float v;
      if constexpr (BF16) v = __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(base)[src + d] << 16);
      else v = reinterpret_cast<const float*>(base)[src + d];
      xs[i] = v;
    }
    __syncthreads();
    float acc = 0.0f;
    const float* xh = xs + half * D;
#pragma unroll
    for (int i = 0; i < D; i += 4) {
      const float4 x4 = *reinterpret_cast<const float4*>(xh + i);
      acc = fmaf(w1[i], x4.x, acc);
      acc = fmaf(w1[i + 1], x4.y, acc);
      acc = fmaf(w1[i + 2], x4.z, acc);
      acc = fmaf(w1[i + 3], x4.w, acc);
    }
    acc += __shfl_xor(acc, 32);
    float hv = fmaxf(acc + b1, 0.0f) * w2;
#pragma unroll
    for (int o = 1; o < 32; o <<= 1) hv += __shfl_xor(hv, o);
    if (lane == 0) p.scores[((size_t)b * p.hkv + h) * p.max_ctx + pos] = hv + b2;
  }
}

// ----------------------------------------------------------------- top-k
struct TopkParams {
  const float* scores;
  const int32_t* seq_lens;
  uint32_t* mask;
  int hkv;
  int max_ctx;
  int words;
  int budget;
};

// Order-preserving key: larger score -> larger key; NaN -> 0 (below -inf); -0 == +0.
__device__ inline uint32_t order_key(float f) {
  if (f != f) return 0u;
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

constexpr int kTopkThreads = 1024;

__global__ __launch_bounds__(kTopkThreads) void topk_kernel(TopkParams p) {
  __shared__ uint32_t hist[256];
  __shared__ uint32_t scan[kTopkThreads / 64];
  __shared__ uint32_t sel_digit, sel_above;
  const int h = blockIdx.x;
  const int b = blockIdx.y;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;
  int L = p.seq_lens[b];
  if (L < 0) L = 0;
  if (L > p.max_ctx) L = p.max_ctx;
  const int n4 = L > kInt8Slots ? L - kInt8Slots : 0;
  const long long k = ((long long)p.budget * n4) / 1000;
  const float* sc = p.scores + ((size_t)b * p.hkv + h) * p.max_ctx + kSink;
  uint32_t* mrow = p.mask + ((size_t)b * p.hkv + h) * p.words;

  // ---- radix select of the k-th largest key (only when 0 < k < n4)
  uint32_t T = 0xFFFFFFFFu;  // threshold key; with need = 0 nothing at T is kept
  long long need = 0;         // how many keys == T to keep (lowest positions first)
  const bool all = k >= n4;
  if (k > 0 && !all) {
    uint32_t prefix = 0, pmask = 0;
    long long remaining = k;
    for (int pass = 0; pass < 4; ++pass) {
      const int shift = 24 - 8 * pass;
      for (int i = tid; i < 256; i += kTopkThreads) hist[i] = 0;
      __syncthreads();
      // 16 scores per thread per step, all loads issued before any is used
      for (int base = tid; base < n4; base += kTopkThreads * 16) {
        float v[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          const int i = base + u * kTopkThreads;
          v[u] = i < n4 ? sc[i] : 0.0f;
        }
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          if (base + u * kTopkThreads < n4) {
            const uint32_t key = order_key(v[u]);
            if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
          }
        }
      }
      __syncthreads();
      if (wid == 0) {
        // lane l owns bins 4l..4l+3; suffix sums from the top bin down
        uint32_t c0 = hist[4 * lane], c1 = hist[4 * lane + 1], c2 = hist[4 * lane + 2],
                 c3 = hist[4 * lane + 3];
        const uint32_t s = c0 + c1 + c2 + c3;
        uint32_t suf = s;  // inclusive suffix over lanes >= lane
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          const uint32_t t = __shfl_down(suf, o);
          if (lane + o < 64) suf += t;
        }
        const uint32_t above = suf - s;  // keys in bins of higher lanes
        if ((long long)above < remaining && remaining <= (long long)suf) {
          uint32_t acc = above;
          int d = 4 * lane + 3;
          const uint32_t cs[4] = {c0, c1, c2, c3};
          for (int q = 3; q >= 0; --q) {
            if ((long long)(acc + cs[q]) >= remaining) { d = 4 * lane + q; break; }
            acc += cs[q];
          }
          sel_digit = (uint32_t)d;
          sel_above = acc;
        }
      }
      __syncthreads();
      const uint32_t d = sel_digit;
      remaining -= sel_above;
      prefix |= d << shift;
      pmask |= 255u << shift;
      __syncthreads();
    }
    T = prefix;
    need = remaining;
  }

  // ---- in-order pass: one mask word per thread, block-wide running count of keys == T
  long long carry = 0;
  for (int w0 = 0; w0 < p.words; w0 += kTopkThreads) {
    const int w = w0 + tid;
    uint32_t gt = 0, eq = 0;  // bit masks over the word's INT4 positions
    if (w < p.words && k > 0 && !all) {
      float v[32];
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        const int t = w * 32 + i;
        v[i] = (t >= kSink && t < kSink + n4) ? sc[t - kSink] : 0.0f;
      }
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        const int t = w * 32 + i;
        if (t >= kSink && t < kSink + n4) {
          const uint32_t key = order_key(v[i]);
          if (key > T) gt |= 1u << i;
          else if (key == T) eq |= 1u << i;
        }
      }
    }
    // exclusive prefix (in word order) of popcount(eq) across the block
    uint32_t cnt = __popc(eq);
    uint32_t incl = cnt;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const uint32_t t = __shfl_up(incl, o);
      if (lane >= o) incl += t;
    }
    if (lane == 63) scan[wid] = incl;
    __syncthreads();
    uint32_t wave_base = 0, tile_total = 0;
    for (int q = 0; q < kTopkThreads / 64; ++q) {
      const uint32_t v = scan[q];
      if (q < wid) wave_base += v;
      tile_total += v;
    }
    const long long before = carry + wave_base + (incl - cnt);
    if (w < p.words) {
      uint32_t bits = gt;
      if (eq) {
        long long r = before;
        for (int i = 0; i < 32; ++i) {
          if (eq & (1u << i)) {
            if (r < need) bits |= 1u << i;
            ++r;
          }
        }
      }
      // protected positions are always kept; INT4 fully kept when k == n4
      for (int i = 0; i < 32; ++i) {
        const int t = w * 32 + i;
        if (t >= L) { bits &= ~(1u << i); continue; }
        const bool prot = t < kSink || t >= L - kRecent;
        if (prot || (all && t >= kSink)) bits |= 1u << i;
      }
      mrow[w] = bits;
    }
    carry += tile_total;
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_score(const kvc_cache& c, const float* mlp, const void* k_new, const void* v_new,
                        kvc_dtype src, int n_new_max, const int32_t* n_new, hipStream_t s) {
  ScoreParams p;
  p.mlp = mlp;
  p.k_new = k_new;
  p.v_new = v_new;
  p.n_new = n_new;
  p.seq_lens = c.seq_lens;
  p.scores = c.scores;
  p.batch = c.batch;
  p.hkv = c.num_kv_heads;
  p.n_new_max = n_new_max;
  p.max_ctx = c.max_ctx;
  const long long total = (long long)c.batch * n_new_max;
  long long tpw = (total + 511) / 512;
  if (tpw < 16) tpw = 16;
  p.tokens_per_wave = (int)tpw;
  p.waves_per_head = (int)((total + tpw - 1) / tpw);
  const dim3 grid((unsigned)(p.waves_per_head * c.num_kv_heads));
  const bool bf = src == KVC_BF16;
  if (c.head_dim == 128) {
    if (bf) hipLaunchKernelGGL((score_kernel<128, true>), grid, dim3(64), 0, s, p);
    else hipLaunchKernelGGL((score_kernel<128, false>), grid, dim3(64), 0, s, p);
  } else {
    if (bf) hipLaunchKernelGGL((score_kernel<64, true>), grid, dim3(64), 0, s, p);
    else hipLaunchKernelGGL((score_kernel<64, false>), grid, dim3(64), 0, s, p);
  }
  return hipGetLastError();
}

hipError_t launch_topk(const kvc_cache& c, int budget_permille, hipStream_t s) {
  TopkParams p;
  p.scores = c.scores;
  p.seq_lens = c.seq_lens;
  p.mask = c.keep_mask;
  p.hkv = c.num_kv_heads;
  p.max_ctx = c.max_ctx;
  p.words = mask_words(c.max_ctx);
  p.budget = budget_permille;
  hipLaunchKernelGGL(topk_kernel, dim3(c.num_kv_heads, c.batch), dim3(kTopkThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace kvc
