// Temporal tiering of the INT4 pages (TTKV promo page, arXiv 2604.19769,
// strengths section: a temporal-tiered cache keeps hot data in HBM and cold
// data in DRAM):
// the caller moves pages between the device pool and a host pool in pinned
// memory with these two helpers and rewrites the block table; attention and
// the append read and write pages of either tier in place.
//   find_pages: logical pages that are demotion candidates (device tier, all
//               16 positions in the INT4 region and evicted for every kv head)
//               or promotion candidates (host tier, some position kept).
//   copy_pages: whole-page copies (codes and meta of every kv head) between
//               physical pages of either tier.

#include "kvc_internal.h"

namespace kvc {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

struct TierParams {
  const int32_t* block_table;
  const int32_t* seq_lens;
  const uint32_t* mask;
  int batch, hkv, max_pages, words, max_ctx, num_pages, host_pages, sink, recent;
};

__global__ void zero_count_kernel(int32_t* count) {
  if (threadIdx.x == 0) *count = 0;
}

// One thread per (sequence, logical page).
__global__ __launch_bounds__(256) void find_pages_kernel(TierParams p, int mode, int32_t* out, int cap,
                                                         int32_t* count) {
  const long long t = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= (long long)p.batch * p.max_pages) return;
  const int b = (int)(t / p.max_pages), lp = (int)(t % p.max_pages);
  int L = p.seq_lens[b];
  L = L < 0 ? 0 : (L > p.max_ctx ? p.max_ctx : L);
  const int t0 = kPage * lp;
  if (t0 >= L) return;
  const int page = p.block_table[(size_t)b * p.max_pages + lp];
  if (page < 0 || page >= p.num_pages + p.host_pages) return;
  // the page's 16 mask bits of every kv head (16-position pages, 32-bit words)
  uint32_t any = 0;
  for (int h = 0; h < p.hkv; ++h) {
    const uint32_t w = p.mask[((size_t)b * p.hkv + h) * p.words + (t0 >> 5)];
    any |= (w >> (t0 & 31)) & 0xFFFFu;
  }
  bool pick;
  if (mode == 0) {
    const bool int4_only = t0 >= p.sink && t0 + kPage <= L - p.recent;
    pick = page < p.num_pages && int4_only && any == 0;
  } else {
    pick = page >= p.num_pages && any != 0;
  }
  if (pick) {
    const int at = atomicAdd(count, 1);
    if (at < cap) {
      out[2 * at] = b;
      out[2 * at + 1] = lp;
    }
  }
}

struct CopyParams {
  uint8_t* codes;
  uint16_t* meta;
  uint8_t* codes_h;
  uint16_t* meta_h;
  const int32_t* src;
  const int32_t* dst;
  int n, num_pages, host_pages;
  size_t code_bytes, meta_bytes;  // per physical page (all kv heads)
};

// One workgroup per page copy, 16-byte pieces.
__global__ __launch_bounds__(256) void copy_pages_kernel(CopyParams p) {
  const int i = blockIdx.x;
  if (i >= p.n) return;
  const int s = p.src[i], d = p.dst[i];
  const int lim = p.num_pages + p.host_pages;
  if (s < 0 || s >= lim || d < 0 || d >= lim || s == d) return;
  auto codes_of = [&](int pg) -> uint8_t* {
    return pg < p.num_pages ? p.codes + (size_t)pg * p.code_bytes
                            : p.codes_h + (size_t)(pg - p.num_pages) * p.code_bytes;
  };
  auto meta_of = [&](int pg) -> uint8_t* {
    return pg < p.num_pages
               ? reinterpret_cast<uint8_t*>(p.meta) + (size_t)pg * p.meta_bytes
               : reinterpret_cast<uint8_t*>(p.meta_h) + (size_t)(pg - p.num_pages) * p.meta_bytes;
  };
  const u32x4* cs = reinterpret_cast<const u32x4*>(codes_of(s));
  u32x4* cd = reinterpret_cast<u32x4*>(codes_of(d));
  for (size_t x = threadIdx.x; x < p.code_bytes / 16; x += blockDim.x) cd[x] = cs[x];
  const u32x4* ms = reinterpret_cast<const u32x4*>(meta_of(s));
  u32x4* md = reinterpret_cast<u32x4*>(meta_of(d));
  for (size_t x = threadIdx.x; x < p.meta_bytes / 16; x += blockDim.x) md[x] = ms[x];
}

}  // namespace

hipError_t launch_find_pages(const kvc_cache& c, int mode, int32_t* out, int cap, int32_t* count,
                             hipStream_t s) {
  TierParams p;
  p.block_table = c.block_table;
  p.seq_lens = c.seq_lens;
  p.mask = c.keep_mask;
  p.batch = c.batch;
  p.hkv = c.num_kv_heads;
  p.max_pages = c.max_pages_per_seq;
  p.words = mask_words(c.max_ctx);
  p.max_ctx = c.max_ctx;
  p.num_pages = c.num_phys_pages;
  p.host_pages = c.num_host_pages;
  p.sink = c.n_sink;
  p.recent = c.n_recent;
  hipLaunchKernelGGL(zero_count_kernel, dim3(1), dim3(64), 0, s, count);
  const long long items = (long long)c.batch * c.max_pages_per_seq;
  hipLaunchKernelGGL(find_pages_kernel, dim3((unsigned)((items + 255) / 256)), dim3(256), 0, s, p,
                     mode, out, cap, count);
  return hipGetLastError();
}

hipError_t launch_copy_pages(const kvc_cache& c, const int32_t* src, const int32_t* dst, int n,
                             hipStream_t s) {
  CopyParams p;
  p.codes = c.int4_codes;
  p.meta = c.int4_meta;
  p.codes_h = c.int4_codes_host;
  p.meta_h = c.int4_meta_host;
  p.src = src;
  p.dst = dst;
  p.n = n;
  p.num_pages = c.num_phys_pages;
  p.host_pages = c.num_host_pages;
  p.code_bytes = (size_t)c.num_kv_heads * kPage * c.head_dim;          // K and V codes
  p.meta_bytes = (size_t)c.num_kv_heads * kPage * (c.head_dim / 32) * 2 * 2 * 2;  // fp16 (scale, min), K and V
  hipLaunchKernelGGL(copy_pages_kernel, dim3((unsigned)n), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace kvc
