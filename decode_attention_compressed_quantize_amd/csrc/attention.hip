// Split-region decode attention over the compressed cache, and the exact
// log-sum-exp merge.
//
// Source: KV4-RL review, section 3 - the INT4 region and the protected INT8
// region are processed independently and their outputs are combined by an
// exact softmax merge, so the full-precision cache is never rebuilt; the
// protected region uses high-fidelity probability-value arithmetic, read here
// as float32 P and float32 decoded V.
//
// Every work item writes an unnormalised partial (m, l, o[D]) per query head:
// m is the running max of the logits in log2 units (logit * log2(e)),
// l = sum 2^(s - m), o = sum 2^(s - m) * v. Item j < nsplit covers INT4 chunk
// j of the sequence's INT4 region; item nsplit covers the INT8 region.
// The merge kernel combines the nsplit + 1 partials in index order, so the
// result does not depend on scheduling.
#include "kvc_internal.h"

namespace kvc {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct AttnParams {
  const void* q;
  const uint8_t* codes;
  const uint16_t* meta;
  const int8_t* codes8;
  const float* scales8;
  const int32_t* block_table;
  const int32_t* seq_lens;
  const uint32_t* mask;
  float* ws;
  float* out;
  float* lse;
  float qscale;  // softmax scale * log2(e)
  int hkv;
  int hq;
  int max_pages;
  int num_pages;
  int max_ctx;
  int words;
  int chunk;
  int nsplit;
};

__device__ inline float h2f(uint16_t b) { return (float)__builtin_bit_cast(_Float16, b); }

__device__ inline float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ inline float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

template <int D, int G, bool QBF16>
__device__ inline void stage_q(const AttnParams& p, int b, int h, float (*qs)[D]) {
  const int lane = threadIdx.x & 63;
  for (int i = lane; i < G * D; i += 64) {
    const int g = i / D, d = i % D;
    const size_t off = ((size_t)b * p.hq + h * G + g) * D + d;
    float v;
    if constexpr (QBF16) v = __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(p.q)[off] << 16);
    else v = reinterpret_cast<const float*>(p.q)[off];
    qs[g][d] = v * p.qscale;
  }
}

template <int D, int G>
__device__ inline void write_partial(const AttnParams& p, int b, int h, int split, const float* m,
                                     const float* l, const float (*o)[D / 64]) {
  constexpr int CPL = D / 64;
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int g = 0; g < G; ++g) {
    float* dst = p.ws + (((size_t)b * p.hq + h * G + g) * (p.nsplit + 1) + split) * (2 + D);
    if (lane == 0) { dst[0] = m[g]; dst[1] = l[g]; }
#pragma unroll
    for (int c = 0; c < CPL; ++c) dst[2 + lane * CPL + c] = o[g][c];
  }
}

// ------------------------------------------------------------------ INT4 region
// One wave per (split, kv head, sequence). Lane = token for the logits (64
// tokens per step); lane = channel(s) for P.V, reading the step's V codes and
// meta from LDS.
template <int D, int G, bool QBF16>
__global__ __launch_bounds__(64) void int4_partial_kernel(AttnParams p) {
  constexpr int CPL = D / 64;     // channels per lane in P.V (2 at D=128, 1 at D=64)
  constexpr int NG = D / 32;      // groups per row
  __shared__ float qs[G][D];
  __shared__ float ps[G][64];
  __shared__ uint8_t vc[64][D / 2];
  __shared__ float vm[64][NG][2];
  const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x;
  int L = p.seq_lens[b];
  L = L < 0 ? 0 : (L > p.max_ctx ? p.max_ctx : L);
  const int n4 = L > kInt8Slots ? L - kInt8Slots : 0;
  const int start = kSink + split * p.chunk;
  const int end = min(kSink + n4, start + p.chunk);
  float m[G], l[G], o[G][CPL];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m[g] = -INFINITY; l[g] = 0.0f;
#pragma unroll
    for (int c = 0; c < CPL; ++c) o[g][c] = 0.0f;
  }
  if (start >= end) { write_partial<D, G>(p, b, h, split, m, l, o); return; }
  stage_q<D, G, QBF16>(p, b, h, qs);
  __syncthreads();
  // per-group sums of q for the min term: qsum[g][grp]
  float qsum[G][NG];
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int k = 0; k < NG; ++k) {
      float s = 0.0f;
      for (int i = 0; i < 32; ++i) s += qs[g][k * 32 + i];
      qsum[g][k] = s;
    }
  const uint32_t* mrow = p.mask + ((size_t)b * p.hkv + h) * p.words;
  const int32_t* bt = p.block_table + (size_t)b * p.max_pages;

  for (int t0 = start; t0 < end; t0 += 64) {
    const int pos = t0 + lane;
    bool valid = pos < end && ((mrow[pos >> 5] >> (pos & 31)) & 1u);
    size_t rec = 0;
    if (valid) {
      const int page = bt[pos / kPage];
      valid = page >= 0 && page < p.num_pages;
      rec = ((size_t)page * p.hkv + h) * kPage + (pos & (kPage - 1));
    }
    float s[G];
#pragma unroll
    for (int g = 0; g < G; ++g) s[g] = -INFINITY;
    if (valid) {
      const uint8_t* kc = p.codes + rec * D;
      const uint16_t* mt = p.meta + rec * NG * 4;
#pragma unroll
      for (int g = 0; g < G; ++g) s[g] = 0.0f;
#pragma unroll
      for (int k = 0; k < NG; ++k) {
        const float ks = h2f(mt[k * 4 + 0]), km = h2f(mt[k * 4 + 1]);
        float dot[G];
#pragma unroll
        for (int g = 0; g < G; ++g) dot[g] = 0.0f;
        for (int i = 0; i < 16; ++i) {
          const uint32_t byte = kc[k * 16 + i];
          const float c0 = (float)(byte & 15u), c1 = (float)(byte >> 4);
#pragma unroll
          for (int g = 0; g < G; ++g)
            dot[g] += qs[g][k * 32 + 2 * i] * c0 + qs[g][k * 32 + 2 * i + 1] * c1;
        }
#pragma unroll
        for (int g = 0; g < G; ++g) s[g] += ks * dot[g] + km * qsum[g][k];
      }
      // stage V codes and meta for the P.V pass
      const uint8_t* vcs = kc + D / 2;
      for (int i = 0; i < D / 2; ++i) vc[lane][i] = vcs[i];
#pragma unroll
      for (int k = 0; k < NG; ++k) { vm[lane][k][0] = h2f(mt[k * 4 + 2]); vm[lane][k][1] = h2f(mt[k * 4 + 3]); }
    } else {
      for (int i = 0; i < D / 2; ++i) vc[lane][i] = 0;
#pragma unroll
      for (int k = 0; k < NG; ++k) { vm[lane][k][0] = 0.0f; vm[lane][k][1] = 0.0f; }
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float mb = wave_max(s[g]);
      const float mn = fmaxf(m[g], mb);
      float pg = 0.0f;
      if (mn != -INFINITY) {
        const float alpha = m[g] == -INFINITY ? 0.0f : exp2f(m[g] - mn);
        pg = valid ? exp2f(s[g] - mn) : 0.0f;
        l[g] = l[g] * alpha + pg;
#pragma unroll
        for (int c = 0; c < CPL; ++c) o[g][c] *= alpha;
        m[g] = mn;
      }
      ps[g][lane] = pg;
    }
    __syncthreads();
    const int nt = min(64, end - t0);
    for (int j = 0; j < nt; ++j) {
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        const int ch = lane * CPL + c;
        const uint32_t byte = vc[j][ch >> 1];
        const float code = (float)((ch & 1) ? (byte >> 4) : (byte & 15u));
        const float v = code * vm[j][ch >> 5][0] + vm[j][ch >> 5][1];
#pragma unroll
        for (int g = 0; g < G; ++g) o[g][c] += ps[g][j] * v;
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int g = 0; g < G; ++g) l[g] = wave_sum(l[g]);
  write_partial<D, G>(p, b, h, split, m, l, o);
}

// ------------------------------------------------------------------ INT8 region
// One wave per (kv head, sequence) over the <= 144 protected positions, all in
// float32: logits from int8 codes times the K scale, P.V with decoded V.
template <int D, int G, bool QBF16>
__global__ __launch_bounds__(64) void int8_partial_kernel(AttnParams p) {
  constexpr int CPL = D / 64;
  __shared__ float qs[G][D];
  __shared__ float ps[G][64];
  __shared__ float vv[64][D];
  const int h = blockIdx.x, b = blockIdx.y;
  const int lane = threadIdx.x;
  int L = p.seq_lens[b];
  L = L < 0 ? 0 : (L > p.max_ctx ? p.max_ctx : L);
  const int ns = L < kSink ? L : kSink;
  const int r0 = L - kRecent > kSink ? L - kRecent : kSink;  // first recent position
  const int nr = L > r0 ? L - r0 : 0;
  const int n8 = ns + nr;
  float m[G], l[G], o[G][CPL];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m[g] = -INFINITY; l[g] = 0.0f;
#pragma unroll
    for (int c = 0; c < CPL; ++c) o[g][c] = 0.0f;
  }
  if (n8 == 0) { write_partial<D, G>(p, b, h, p.nsplit, m, l, o); return; }
  stage_q<D, G, QBF16>(p, b, h, qs);
  __syncthreads();
  const size_t base = ((size_t)b * p.hkv + h) * kInt8Slots;
  for (int i0 = 0; i0 < n8; i0 += 64) {
    const int i = i0 + lane;
    const bool valid = i < n8;
    float s[G];
#pragma unroll
    for (int g = 0; g < G; ++g) s[g] = -INFINITY;
    if (valid) {
      const int pos = i < ns ? i : r0 + (i - ns);
      const int slot = pos < kSink ? pos : kSink + (pos - kSink) % kRecent;
      const int8_t* kc = p.codes8 + (base + slot) * 2 * D;
      const float ks = p.scales8[(base + slot) * 2 + 0];
      const float vs = p.scales8[(base + slot) * 2 + 1];
      float dot[G];
#pragma unroll
      for (int g = 0; g < G; ++g) dot[g] = 0.0f;
      for (int d = 0; d < D; ++d) {
        const float c = (float)kc[d];
#pragma unroll
        for (int g = 0; g < G; ++g) dot[g] += qs[g][d] * c;
      }
#pragma unroll
      for (int g = 0; g < G; ++g) s[g] = ks * dot[g];
      for (int d = 0; d < D; ++d) vv[lane][d] = (float)kc[D + d] * vs;
    } else {
      for (int d = 0; d < D; ++d) vv[lane][d] = 0.0f;
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float mb = wave_max(s[g]);
      const float mn = fmaxf(m[g], mb);
      float pg = 0.0f;
      if (mn != -INFINITY) {
        const float alpha = m[g] == -INFINITY ? 0.0f : exp2f(m[g] - mn);
        pg = valid ? exp2f(s[g] - mn) : 0.0f;
        l[g] = l[g] * alpha + pg;
#pragma unroll
        for (int c = 0; c < CPL; ++c) o[g][c] *= alpha;
        m[g] = mn;
      }
      ps[g][lane] = pg;
    }
    __syncthreads();
    const int nt = min(64, n8 - i0);
    for (int j = 0; j < nt; ++j)
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        const float v = vv[j][lane * CPL + c];
#pragma unroll
        for (int g = 0; g < G; ++g) o[g][c] += ps[g][j] * v;
      }
    __syncthreads();
  }
#pragma unroll
  for (int g = 0; g < G; ++g) l[g] = wave_sum(l[g]);
  write_partial<D, G>(p, b, h, p.nsplit, m, l, o);
}

// ------------------------------------------------------------------ merge
// One wave per (query head, sequence): out = sum_j w_j o_j / sum_j w_j l_j with
// w_j = 2^(m_j - M); lse = ln 2 * (M + log2 sum_j w_j l_j).
template <int D>
__global__ __launch_bounds__(64) void merge_kernel(AttnParams p) {
  constexpr int CPL = D / 64;
  const int hq = blockIdx.x, b = blockIdx.y;
  const int lane = threadIdx.x;
  const int np = p.nsplit + 1;
  const float* parts = p.ws + ((size_t)b * p.hq + hq) * np * (2 + D);
  float M = -INFINITY;
  for (int j = 0; j < np; ++j) M = fmaxf(M, parts[(size_t)j * (2 + D)]);
  float den = 0.0f, num[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) num[c] = 0.0f;
  if (M != -INFINITY) {
    for (int j = 0; j < np; ++j) {
      const float* pj = parts + (size_t)j * (2 + D);
      const float mj = pj[0];
      if (mj == -INFINITY) continue;
      const float w = exp2f(mj - M);
      den += w * pj[1];
#pragma unroll
      for (int c = 0; c < CPL; ++c) num[c] += w * pj[2 + lane * CPL + c];
    }
  }
  float* o = p.out + ((size_t)b * p.hq + hq) * D;
  const float inv = den > 0.0f ? 1.0f / den : 0.0f;
#pragma unroll
  for (int c = 0; c < CPL; ++c) o[lane * CPL + c] = num[c] * inv;
  if (p.lse && lane == 0)
    p.lse[(size_t)b * p.hq + hq] = den > 0.0f ? (M + log2f(den)) * kLn2 : -INFINITY;
}

template <int D, int G, bool QBF16>
hipError_t launch_all(const kvc_cache& c, const AttnParams& p, hipStream_t s) {
  hipLaunchKernelGGL((int4_partial_kernel<D, G, QBF16>), dim3(p.nsplit, c.num_kv_heads, c.batch),
                     dim3(64), 0, s, p);
  hipLaunchKernelGGL((int8_partial_kernel<D, G, QBF16>), dim3(c.num_kv_heads, c.batch), dim3(64), 0,
                     s, p);
  hipLaunchKernelGGL((merge_kernel<D>), dim3(p.hq, c.batch), dim3(64), 0, s, p);
  return hipGetLastError();
}

template <int D, int G>
hipError_t launch_dq(const kvc_cache& c, const AttnParams& p, bool qbf16, hipStream_t s) {
  return qbf16 ? launch_all<D, G, true>(c, p, s) : launch_all<D, G, false>(c, p, s);
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
  p.ws = ws;
  p.out = out;
  p.lse = lse;
  p.qscale = softmax_scale * kLog2e;
  p.hkv = c.num_kv_heads;
  p.hq = num_q_heads;
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
      case 8: return launch_dq<64, 8>(c, p, bf, s);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace kvc
