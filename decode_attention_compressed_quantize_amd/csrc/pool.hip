// Kept-record pool rebuilt from the keep mask (kvc_pool_build), for masks the
// caller wrote itself; the top-k refresh maintains the pool on its own.
//
// Source: Shadow Mask Distillation page, Figure 1 caption - the mask of
// retained indices decides what is attended; KV4-RL review, section 3 - those
// positions are read from the INT4 store. The pool is a compact copy of
// exactly those records (layout in pool_layout.h).
//
// One 256-thread workgroup per (sequence, kv head, run of 256 mask words):
// thread t owns one mask word; the records of its kept INT4-region positions
// (pages outside the pools skipped) go to slots numbered in position order,
// so the workgroup first counts the kept positions of every earlier word.
#include "kvc_internal.h"
#include "pool_layout.h"

namespace kvc {
namespace {

constexpr int kBuildThreads = 256;

struct BuildParams {
  PoolRef pool;
  const uint32_t* mask;
  const int32_t* seq_lens;
  int words;
  int sink, recent;
};

// Kept INT4-region bits of mask word w (positions 32w..32w+31) whose page is
// valid, for a sequence with INT4 region [r0, r1); pages returned for the copy.
__device__ inline uint32_t kept_bits(const BuildParams& p, int b, const uint32_t* mrow, int w, int r0,
                                     int r1, int& pga, int& pgb, bool report) {
  pga = pgb = -1;
  const int lo = r0 - 32 * w, hi = r1 - 32 * w;
  if (hi <= 0 || lo >= 32) return 0u;
  uint32_t k4 = mrow[w];
  if (lo > 0) k4 &= ~0u << lo;
  if (hi < 32) k4 &= (1u << hi) - 1u;
  const int32_t* bt = p.pool.block_table + (size_t)b * p.pool.max_pages;
  const int lim = p.pool.num_pages + p.pool.host_pages;
  if (k4 & 0x0000FFFFu) {
    pga = bt[2 * w];
    if (pga < 0 || pga >= lim) {
      k4 &= 0xFFFF0000u;
      if (report) report_error(p.pool.errors, KVC_ERR_PAGE);
    }
  }
  if (k4 & 0xFFFF0000u) {
    pgb = bt[2 * w + 1];
    if (pgb < 0 || pgb >= lim) {
      k4 &= 0x0000FFFFu;
      if (report) report_error(p.pool.errors, KVC_ERR_PAGE);
    }
  }
  return k4;
}

__device__ inline uint32_t block_sum(uint32_t v, uint32_t* red) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  if (lane == 0) red[wid] = v;
  __syncthreads();
  uint32_t t = 0;
#pragma unroll
  for (int q = 0; q < kBuildThreads / 64; ++q) t += red[q];
  __syncthreads();
  return t;
}

__global__ __launch_bounds__(kBuildThreads) void pool_build_kernel(BuildParams p) {
  __shared__ uint32_t red[kBuildThreads / 64];
  __shared__ uint32_t scan[kBuildThreads / 64];
  const int pair = blockIdx.y;
  const int b = pair / p.pool.hkv, h = pair % p.pool.hkv;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  int L = p.seq_lens[b];
  if (L < 0 || L > p.pool.max_ctx) {
    if (tid == 0 && blockIdx.x == 0) report_error(p.pool.errors, KVC_ERR_LENGTH);
    L = L < 0 ? 0 : p.pool.max_ctx;
  }
  const int slots = p.sink + p.recent;
  const int n4 = L > slots ? L - slots : 0;
  const int r0 = p.sink, r1 = p.sink + n4;
  const int wlast = n4 > 0 ? (r1 - 1) >> 5 : 0;  // last word holding INT4-region positions
  const int w0 = blockIdx.x * kBuildThreads;
  if (w0 > wlast) return;
  const uint32_t* mrow = p.mask + (size_t)pair * p.words;
  // kept records in the words before this run
  uint32_t before = 0;
  for (int w = tid; w < w0; w += kBuildThreads) {
    int a, c;
    before += __popc(kept_bits(p, b, mrow, w, r0, r1, a, c, false));
  }
  before = block_sum(before, red);
  // this run: one word per thread, slots in position order
  const int w = w0 + tid;
  int pga = -1, pgb = -1;
  uint32_t k4 = w <= wlast ? kept_bits(p, b, mrow, w, r0, r1, pga, pgb, true) : 0u;
  const uint32_t pc = (uint32_t)__popc(k4);
  uint32_t incl = pc;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t t = __shfl_up(incl, o);
    if (lane >= o) incl += t;
  }
  if (lane == 63) scan[wid] = incl;
  __syncthreads();
  uint32_t wave_base = 0, total = 0;
#pragma unroll
  for (int q = 0; q < kBuildThreads / 64; ++q) {
    if (q < wid) wave_base += scan[q];
    total += scan[q];
  }
  long long slot = (long long)before + wave_base + (incl - pc);
  bool over = false;
  while (k4 != 0) {
    const int bit = __builtin_ctz(k4);
    k4 &= k4 - 1u;
    const int pos = 32 * w + bit;
    if (slot < p.pool.cap) {
      pool_copy_thread(p.pool, pair, h, bit < 16 ? pga : pgb, pos, (int)slot);
      pool_slot_of(p.pool, pair)[pos] = (int32_t)slot;
      pool_pos_of(p.pool, pair)[slot] = pos;
    } else {
      over = true;
    }
    ++slot;
  }
  if (over) report_error(p.pool.errors, KVC_ERR_POOL);
  // the run holding the region's last word writes the header
  if (tid == 0 && (int)blockIdx.x == wlast / kBuildThreads) {
    const long long count = (long long)before + total;
    const bool fits = count <= p.pool.cap;
    int32_t* hdr = p.pool.header + 4 * (size_t)pair;
    hdr[0] = (int32_t)(fits ? count : p.pool.cap);
    hdr[1] = L;
    hdr[2] = fits ? (int32_t)kPoolMagic : 0;
    hdr[3] = 0;
  }
}

}  // namespace

hipError_t launch_pool_build(const kvc_cache& c, hipStream_t s) {
  BuildParams p;
  p.pool = pool_ref(c);
  p.mask = c.keep_mask;
  p.seq_lens = c.seq_lens;
  p.words = mask_words(c.max_ctx);
  p.sink = c.n_sink;
  p.recent = c.n_recent;
  const dim3 grid((unsigned)((p.words + kBuildThreads - 1) / kBuildThreads),
                  (unsigned)(c.batch * c.num_kv_heads));
  hipLaunchKernelGGL(pool_build_kernel, grid, dim3(kBuildThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace kvc
