// Quantize-on-append of one (sequence, appended token, kv head): INT4 for
// every appended position, INT8 for the sink and recent-window positions of
// the new length. Shared by the append launch and the fused append + score +
// refresh launch, so both write the same bytes.
//
// Source: KV4-RL review, section 3 - the full context is stored as paged,
// calibration-free INT4 and the first 16 and the 128 most recent positions
// are also kept in an INT8 side cache. The numeric rule (group 32, fp16
// scale/min, per-token absmax INT8, round-to-nearest-even float32 steps) is
// the one stated in kvc.h: every product and difference rounds on its own
// (no contraction into fused multiply-adds inside quantize_item).
//
// One wave encodes one item: lanes 0-31 take K, lanes 32-63 take V, D/32
// consecutive elements per lane, so a 32-wide group spans 32/(D/32) lanes and
// its min/max is a short xor-shuffle tree.
#pragma once
#include "kvc_internal.h"

namespace kvc {

struct QuantParams {
  const void* k_new;
  const void* v_new;
  const int32_t* n_new;
  const int32_t* seq_lens;
  const int32_t* block_table;
  uint8_t* codes;
  uint16_t* meta;
  int8_t* codes8;
  float* scales8;
  long long items;  // B * n_new_max * Hkv
  int n_new_max;
  int hkv;
  int max_pages;
  int num_pages;
  int max_ctx;
  int sink, recent;
  uint8_t* codes_h;  // host tier: pages [num_pages, num_pages + host_pages)
  uint16_t* meta_h;
  int host_pages;  // INT8-protected sink and recent positions (16/128, or 0/0)
  // kept-record pool headers [B][Hkv][4], or null: rows that rewrite INT4
  // records the pool may hold clear its validity word
  int32_t* pool_header;
};

__device__ inline float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

template <int EPL, bool BF16>
__device__ inline void load_elems(const void* base, size_t off, float (&x)[EPL]) {
  if constexpr (BF16) {
    const uint16_t* p = reinterpret_cast<const uint16_t*>(base) + off;
    if constexpr (EPL == 4) {
      uint2 u = *reinterpret_cast<const uint2*>(p);
      x[0] = __uint_as_float(u.x << 16);
      x[1] = __uint_as_float(u.x & 0xFFFF0000u);
      x[2] = __uint_as_float(u.y << 16);
      x[3] = __uint_as_float(u.y & 0xFFFF0000u);
    } else {
      uint32_t u = *reinterpret_cast<const uint32_t*>(p);
      x[0] = __uint_as_float(u << 16);
      x[1] = __uint_as_float(u & 0xFFFF0000u);
    }
  } else {
    const float* p = reinterpret_cast<const float*>(base) + off;
    if constexpr (EPL == 4) {
      float4 f = *reinterpret_cast<const float4*>(p);
      x[0] = f.x; x[1] = f.y; x[2] = f.z; x[3] = f.w;
    } else {
      float2 f = *reinterpret_cast<const float2*>(p);
      x[0] = f.x; x[1] = f.y;
    }
  }
}

__device__ inline uint16_t f16_bits(float v) {
  _Float16 h = (_Float16)v;
  return __builtin_bit_cast(uint16_t, h);
}

inline QuantParams quant_params(const kvc_cache& c, const void* k_new, const void* v_new,
                                int n_new_max, const int32_t* n_new) {
  QuantParams p;
  p.k_new = k_new;
  p.v_new = v_new;
  p.n_new = n_new;
  p.seq_lens = c.seq_lens;
  p.block_table = c.block_table;
  p.codes = c.int4_codes;
  p.meta = c.int4_meta;
  p.codes8 = c.int8_codes;
  p.scales8 = c.int8_scales;
  p.items = (long long)c.batch * n_new_max * c.num_kv_heads;
  p.n_new_max = n_new_max;
  p.hkv = c.num_kv_heads;
  p.max_pages = c.max_pages_per_seq;
  p.num_pages = c.num_phys_pages;
  p.max_ctx = c.max_ctx;
  p.sink = c.n_sink;
  p.recent = c.n_recent;
  p.codes_h = c.int4_codes_host;
  p.meta_h = c.int4_meta_host;
  p.host_pages = c.num_host_pages;
  p.pool_header = nullptr;
  return p;
}

// item = (sequence * n_new_max + appended index) * Hkv + kv head; lane = lane
// of the calling wave (the whole wave must call)
template <int D, bool BF16>
__device__ inline void quantize_item(const QuantParams& p, long long item, int lane) {
#pragma clang fp contract(off)

  constexpr int EPL = D / 32;  // elements per lane
  constexpr int LPG = 32 / EPL;  // lanes per 32-wide group
  if (item >= p.items) return;
  const int h = (int)(item % p.hkv);
  const long long bj = item / p.hkv;
  const int j = (int)(bj % p.n_new_max);
  const int b = (int)(bj / p.n_new_max);
  // The loads that depend on nothing else go out together (the row - every
  // row j < n_new_max lies in the caller's buffer -, the count and the
  // length), then the page and the pool header, so an append costs two
  // memory round trips before its stores.
  const bool is_v = lane >= 32;
  const int hl = lane & 31;
  float x[EPL];
  const size_t src_off = (((size_t)b * p.n_new_max + j) * p.hkv + h) * D + (size_t)hl * EPL;
  load_elems<EPL, BF16>(is_v ? p.v_new : p.k_new, src_off, x);
  const int nn = p.n_new[b];
  const int L = p.seq_lens[b];
  if (j >= nn) return;
  const int pos = L - nn + j;
  if (pos < 0 || pos >= p.max_ctx || L > p.max_ctx) return;
  const int lp = pos / kPage;
  if (lp >= p.max_pages) return;
  const int page = p.block_table[(size_t)b * p.max_pages + lp];
  if (p.pool_header && j == 0 && lane == 0) {
    // a pool describing length H holds records of positions in [sink, H - recent);
    // rows [pos, L) that reach into that range make it stale
    int32_t* ph = p.pool_header + 4 * ((size_t)b * p.hkv + h);
    const int lo = pos > p.sink ? pos : p.sink;
    if (lo < L && lo < ph[1] - p.recent) ph[2] = 0;
  }
  if (page < 0 || page >= p.num_pages + p.host_pages) return;

  // ---- INT4: group min / max over LPG lanes
  float mn = x[0], mx = x[0];
#pragma unroll
  for (int e = 1; e < EPL; ++e) { mn = fminf(mn, x[e]); mx = fmaxf(mx, x[e]); }
#pragma unroll
  for (int o = 1; o < LPG; o <<= 1) {
    mn = fminf(mn, __shfl_xor(mn, o));
    mx = fmaxf(mx, __shfl_xor(mx, o));
  }
  const float s32 = (mx - mn) / 15.0f;
  const uint16_t sh = f16_bits(fminf(fmaxf(s32, -65504.0f), 65504.0f));
  const uint16_t mh = f16_bits(fminf(fmaxf(mn, -65504.0f), 65504.0f));
  const float sf = (float)__builtin_bit_cast(_Float16, sh);
  const float mf = (float)__builtin_bit_cast(_Float16, mh);
  const float inv = sf > 0.0f ? 1.0f / sf : 0.0f;
  uint32_t packed = 0;
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    const float t = (x[e] - mf) * inv;
    const float r = fminf(fmaxf(__builtin_rintf(t), 0.0f), 15.0f);
    packed |= (uint32_t)r << (4 * e);
  }
  const bool host = page >= p.num_pages;  // a page of the host tier
  uint8_t* const codes = host ? p.codes_h : p.codes;
  uint16_t* const meta = host ? p.meta_h : p.meta;
  const size_t rec = (((size_t)(host ? page - p.num_pages : page) * p.hkv + h) * kPage + (pos & (kPage - 1)));
  uint8_t* crow = codes + rec * D + (is_v ? D / 2 : 0);
  if constexpr (EPL == 4) {
    reinterpret_cast<uint16_t*>(crow)[hl] = (uint16_t)packed;
  } else {
    crow[hl] = (uint8_t)packed;
  }
  if ((hl % LPG) == 0) {
    const int g = hl / LPG;
    uint32_t* m = reinterpret_cast<uint32_t*>(meta + ((rec * 2 + (is_v ? 1 : 0)) * (D / 32) + g) * 2);
    *m = (uint32_t)sh | ((uint32_t)mh << 16);
  }

  // ---- INT8 side cache for sink and recent positions of the new length
  if (p.recent > 0 && (pos < p.sink || pos >= L - p.recent)) {
    float a = fabsf(x[0]);
#pragma unroll
    for (int e = 1; e < EPL; ++e) a = fmaxf(a, fabsf(x[e]));
#pragma unroll
    for (int o = 1; o < 32; o <<= 1) a = fmaxf(a, __shfl_xor(a, o));
    const float s = a / 127.0f;
    const float inv8 = s >= 1.17549435e-38f ? 1.0f / s : 0.0f;
    uint32_t q8 = 0;
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      const float r = fminf(fmaxf(__builtin_rintf(x[e] * inv8), -127.0f), 127.0f);
      q8 |= ((uint32_t)(int32_t)r & 0xFFu) << (8 * e);
    }
    const int slot = pos < p.sink ? pos : p.sink + (pos - p.sink) % p.recent;
    const size_t srec = ((size_t)b * p.hkv + h) * (p.sink + p.recent) + slot;
    int8_t* row = p.codes8 + srec * 2 * D + (is_v ? D : 0) + hl * EPL;
    if constexpr (EPL == 4) {
      *reinterpret_cast<uint32_t*>(row) = q8;
    } else {
      *reinterpret_cast<uint16_t*>(row) = (uint16_t)q8;
    }
    if (hl == 0) p.scales8[srec * 2 + (is_v ? 1 : 0)] = s;
  }
}

}  // namespace kvc
