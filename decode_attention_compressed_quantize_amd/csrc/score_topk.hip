// Per-head scoring MLP and budgeted top-k keep mask (the shadow mask).
//
// Sources: KVP promo page (arXiv 2602.10238), section "Core mechanism" - one
// small MLP per attention head reads the K/V vectors and emits a utility
// score per token; deployment is score -> sort -> truncate to the budget.
// Shadow Mask Distillation page (arXiv 2605.06850), Figure 1 caption - the
// eviction records the retained indices in a binary mask.
//
// Scoring: one 256-thread workgroup per (kv head, run of appended rows); each
// thread holds an eighth of one W1 row in registers, so a decode step (one row
// per sequence) scores every row in parallel.
//
// Top-k: one workgroup per (sequence, kv head). An exact radix select over
// order-preserving 32-bit keys (4 passes of 8 bits, MSB first) finds the
// k-th key T and how many keys equal to T must be kept; a final in-order pass
// keeps every key > T and the lowest-position keys == T, which is the unique
// answer under "score descending, then position ascending". Scores are
// static once written, so a decode step (one position joins the INT4 region,
// k grows by at most one) changes at most two candidate bits: with a state in
// the workspace, one wave applies the step exactly from short sorted lists of
// the keys on either side of the threshold, and the full refresh above runs
// only when the state does not apply (first call, new budget, several new
// positions, caller-written scores, a list run dry).
#include "kvc_internal.h"
#include "pool_layout.h"
#include "quant_row.h"

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
  int tokens_per_group;  // appended rows (b, j) handled by one workgroup
  int groups_per_head;
};

constexpr int kScoreThreads = 256;

// Scores appended row f = b * n_new_max + j of kv head h with the 256 threads
// gtid = 0..255 of one group. Every thread of the workgroup must call it the
// same number of times (it holds workgroup barriers); `valid` is false for
// rows past the end. Thread gtid owns hidden unit u = gtid / 8 and the input
// slice part = gtid % 8 (2D/8 entries of K||V); the 8 parts of a unit are
// summed with lane shuffles, then relu, w2 and the sum over the 32 units
// (within each wave, then across the group's 4 waves through LDS).
// The thread's slice of head h's scorer: W1 row u restricted to its part, b1[u], w2[u].
template <int D>
struct ScorerSlice {
  float w1[2 * D / 8];
  float b1, w2, b2;
  __device__ void load(const ScoreParams& p, int h, int gtid) {
    constexpr int IN = 2 * D;
    constexpr int PART = IN / 8;
    const int u = gtid >> 3, part = gtid & 7;
    const float* wh = p.mlp + (size_t)h * mlp_floats(D);
#pragma unroll
    for (int i = 0; i < PART; i += 4) {
      const float4 f4 = *reinterpret_cast<const float4*>(wh + (size_t)u * IN + part * PART + i);
      w1[i] = f4.x; w1[i + 1] = f4.y; w1[i + 2] = f4.z; w1[i + 3] = f4.w;
    }
    b1 = wh[kHidden * IN + u];
    w2 = wh[kHidden * IN + kHidden + u];
    b2 = wh[kHidden * IN + 2 * kHidden];
  }
};

template <int D, bool BF16>
__device__ __attribute__((always_inline)) void score_row(const ScoreParams& p, const ScorerSlice<D>& m, int h, long long f, int gtid,
                          float* xs, float* wsum) {
  constexpr int IN = 2 * D;
  constexpr int PART = IN / 8;
  const int lane = gtid & 63;
  const int part = gtid & 7;
  const long long total = (long long)p.batch * p.n_new_max;
  static_assert(IN <= kScoreThreads, "one input entry per thread");
  int b = 0, pos = -1;
  float v = 0.0f;
  if (f < total) {
    b = (int)(f / p.n_new_max);
    const int j = (int)(f % p.n_new_max);
    // the row's entry (every row j < n_new_max lies in the caller's buffer),
    // the count and the length are loaded together: one memory round trip
    const size_t src = (((size_t)b * p.n_new_max + j) * p.hkv + h) * D;
    if (gtid < IN) {
      const void* base = gtid < D ? p.k_new : p.v_new;
      const int d = gtid < D ? gtid : gtid - D;
      if constexpr (BF16) v = __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(base)[src + d] << 16);
      else v = reinterpret_cast<const float*>(base)[src + d];
    }
    const int nn = p.n_new[b];
    const int L = p.seq_lens[b];
    if (j < nn) {
      pos = L - nn + j;
      if (pos >= p.max_ctx) pos = -1;
    }
  }
  const bool valid = pos >= 0;
  __syncthreads();  // xs and wsum of the previous row are consumed
  if (valid && gtid < IN) xs[gtid] = v;
  __syncthreads();
  float acc = 0.0f;
  if (valid) {
#pragma unroll
    for (int i = 0; i < PART; i += 4) {
      const float4 x4 = *reinterpret_cast<const float4*>(xs + part * PART + i);
      acc = fmaf(m.w1[i], x4.x, acc);
      acc = fmaf(m.w1[i + 1], x4.y, acc);
      acc = fmaf(m.w1[i + 2], x4.z, acc);
      acc = fmaf(m.w1[i + 3], x4.w, acc);
    }
  }
  // the 8 parts of unit u sit in 8 consecutive lanes
  acc += __shfl_xor(acc, 1);
  acc += __shfl_xor(acc, 2);
  acc += __shfl_xor(acc, 4);
  float hv = part == 0 ? fmaxf(acc + m.b1, 0.0f) * m.w2 : 0.0f;
  // 8 units per wave, then the 4 waves
#pragma unroll
  for (int o = 8; o < 64; o <<= 1) hv += __shfl_xor(hv, o);
  if (lane == 0) wsum[gtid >> 6] = hv;
  __syncthreads();
  if (valid && gtid == 0) {
    float sum = 0.0f;
#pragma unroll
    for (int w = 0; w < kScoreThreads / 64; ++w) sum += wsum[w];
    p.scores[((size_t)b * p.hkv + h) * p.max_ctx + pos] = sum + m.b2;
  }
}

// One 256-thread workgroup per (kv head, run of appended rows).
template <int D, bool BF16>
__global__ __launch_bounds__(kScoreThreads) void score_kernel(ScoreParams p) {
  __shared__ float xs[2 * D];
  __shared__ float wsum[kScoreThreads / 64];
  const int h = blockIdx.x / p.groups_per_head;
  const int g = blockIdx.x % p.groups_per_head;
  const long long f0 = (long long)g * p.tokens_per_group;
  ScorerSlice<D> m;
  m.load(p, h, threadIdx.x);
  for (int i = 0; i < p.tokens_per_group; ++i) score_row<D, BF16>(p, m, h, f0 + i, threadIdx.x, xs, wsum);
}

// ----------------------------------------------------------------- top-k
struct TopkParams {
  const float* scores;
  const int32_t* seq_lens;
  uint32_t* mask;
  TopkState* state;  // per (sequence, kv head), or null
  int incremental;   // the caller wrote no score below the previous length
  int hkv;
  int max_ctx;
  int words;
  int budget;
  int sink, recent;  // INT8-protected sink and recent positions (16/128, or 0/0)
  PoolRef pool;      // kept-record pool maintained with the mask (pool.cap = 0: none)
  int group;         // pairs per workgroup: 1, or kTopkGroup for a decode step (topk_group)
  int pairs;         // batch * hkv
};

// Order-preserving key: larger score -> larger key; NaN -> 0 (below -inf); -0 == +0.
__device__ inline uint32_t order_key(float f) {
  if (f != f) return 0u;
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Composite key: score first, then the lower position.
__device__ inline uint64_t comp_key(uint32_t key, int pos) {
  return ((uint64_t)key << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)pos);
}
__device__ inline int comp_pos(uint64_t c) { return (int)(0xFFFFFFFFu - (uint32_t)c); }

constexpr int kTopkThreads = 1024;
constexpr int kTopkGroup = kTopkThreads / 64;  // at most this many pairs per workgroup in a decode step
// Top-k workgroups a decode step aims for: half of the 256 resident 1024-thread
// workgroups (one per CU at 128 VGPRs), leaving the rest of the round to the
// encoding and scoring workgroups of the same launch (measured: 128 against
// 256 and 512 took the uniform step from 75.7 to 70.6 us, the long-tail step
// from 211.8 to 205.1 us and the 36-layer step from 10.04 to 9.87 ms; 64 and
// 32 were no faster)
constexpr int kTopkResident = 128;
constexpr int kCandCap = 512;  // keys around the threshold a refresh can sort into the lists

// ---- one decode step on the lists, one wave, lane i holding a[i] and b[i]
__device__ inline uint64_t wave_at(uint64_t v, int i) {
  return ((uint64_t)__builtin_amdgcn_readlane((int)(v >> 32), i) << 32) |
         (uint32_t)__builtin_amdgcn_readlane((int)v, i);
}
__device__ inline uint64_t from_lane_below(uint64_t v) { return __shfl_up(v, 1); }
__device__ inline uint64_t from_lane_above(uint64_t v) { return __shfl_down(v, 1); }

// Insert x into the ascending list (a) or descending list (b) when it belongs
// to the part the list must hold: always if the list holds its whole side,
// else only if x falls before the list's last entry. A full list drops its
// last entry.
template <bool Ascending>
__device__ inline uint64_t list_insert(uint64_t v, int& n, uint64_t x, bool whole, int lane) {
  if (!whole) {
    if (n == 0) return v;
    const uint64_t last = wave_at(v, n - 1);
    if (Ascending ? !(x < last) : !(x > last)) return v;
  }
  const int at = (int)__popcll(__ballot(lane < n && (Ascending ? v < x : v > x)));
  const uint64_t below = from_lane_below(v);
  n = n < kTopkBuf ? n + 1 : kTopkBuf;
  return lane < at ? v : (lane == at ? x : below);
}
__device__ inline uint64_t list_push_front(uint64_t v, int& n, uint64_t x, int lane) {
  const uint64_t below = from_lane_below(v);
  n = n < kTopkBuf ? n + 1 : kTopkBuf;
  return lane == 0 ? x : below;
}
__device__ inline uint64_t list_pop_front(uint64_t v, int& n) {
  --n;
  return from_lane_above(v);
}

// Applies one appended position (length L - 1 -> L) to the mask and the lists.
// Returns false, having written nothing, when the state does not describe
// length L - 1 under this budget or a list it needs has run out.
__device__ __attribute__((always_inline)) bool topk_step(const TopkParams& p, TopkState* st, int L, int n4, long long k,
                          const float* sc, uint32_t* mrow, int lane, int b, int h) {
  if (L < 1) return false;
  const int slots = p.sink + p.recent;
  const int n4p = L - 1 > slots ? L - 1 - slots : 0;
  const long long kp = ((long long)p.budget * n4p) / 1000;
  const int pair = b * p.hkv + h;
  int32_t* phdr = p.pool.cap > 0 ? p.pool.header + 4 * (size_t)pair : nullptr;
  // Every load the step may need is issued before any decision, so that the
  // step costs about one memory round trip: the state and its lists, the pool
  // header, the entering position's score, and - speculatively - the record
  // of the entering position (the one the pool takes in most steps; its page
  // comes from the table first) and the slot of the smallest kept key (the
  // one an entering key displaces).
  const bool entering = n4 != n4p;
  const int xpos = p.sink + n4p;  // leaves the recent window (or, unprotected, is appended)
  const float sx = entering ? sc[n4p] : 0.0f;
  const uint32_t s_magic = st->magic;
  const int32_t s_len = st->len, s_k = st->k, s_budget = st->budget;
  int na = st->na, nb = st->nb;
  uint64_t A = lane < na ? st->a[lane] : 0, B = lane < nb ? st->b[lane] : 0;  // lane < 64 = kTopkBuf
  int32_t h0 = 0, h1 = 0, h2 = 0;
  if (phdr) {
    h0 = phdr[0];
    h1 = phdr[1];
    h2 = phdr[2];
  }
  int xpage = -1;
  uint4 xrec = make_uint4(0u, 0u, 0u, 0u);
  if (phdr && entering) {
    const int pg = p.pool.block_table[(size_t)b * p.pool.max_pages + (xpos >> 4)];
    if (pg >= 0 && pg < p.pool.num_pages + p.pool.host_pages) {
      xpage = pg;
      if (lane < pool_chunks(p.pool.D))
        xrec = *reinterpret_cast<const uint4*>(pool_src_chunk(p.pool, pg, h, xpos, lane));
    }
  }
  int a0slot = -1;
  if (phdr && na > 0) {
    const int a0pos = (int)comp_pos(wave_at(A, 0));
    if (a0pos >= 0 && a0pos < p.max_ctx) a0slot = pool_slot_of(p.pool, pair)[a0pos];
  }
  if (s_magic != kTopkMagic || s_budget != p.budget || s_len != L - 1 || s_k != kp) return false;
  // the pool must hold exactly the kept records of length L - 1
  if (phdr && (h2 != (int32_t)kPoolMagic || h1 != L - 1 || h0 != kp)) return false;
  int ins_pos = -1, ins_slot = -1;  // pool: the record of ins_pos goes to ins_slot
  if (na < 0 || na > kTopkBuf || nb < 0 || nb > kTopkBuf) return false;
  int clear_pos = -1, set_pos = -1;
  if (entering) {
    const uint64_t x = comp_key(order_key(sx), xpos);
    const long long out_before = n4p - kp;  // candidates not kept
    if (k == n4) {
      // every INT4-region position kept (budget 1000): x joins the kept set;
      // the lists stay empty, as nothing is ever ranked against them
      ins_slot = (int)kp;
      ins_pos = xpos;
    } else if (k == kp) {
      if (k == 0) {
        clear_pos = xpos;
        B = list_insert<false>(B, nb, x, nb == out_before, lane);
      } else {
        if (na == 0) return false;
        const uint64_t a0 = wave_at(A, 0);
        if (x > a0) {  // x displaces the smallest kept key
          clear_pos = comp_pos(a0);
          ins_pos = xpos;
          if (phdr) ins_slot = a0slot;
          const bool whole = na == k;
          A = list_pop_front(A, na);
          B = list_push_front(B, nb, a0, lane);
          A = list_insert<true>(A, na, x, whole, lane);
        } else {
          clear_pos = xpos;
          B = list_insert<false>(B, nb, x, nb == out_before, lane);
        }
      }
    } else {  // one more kept: x or the best key not kept
      ins_slot = (int)kp;  // the pool grows by one record
      if (out_before == 0 || (nb > 0 && x > wave_at(B, 0))) {
        A = list_insert<true>(A, na, x, na == kp, lane);
        ins_pos = xpos;
      } else {
        if (nb == 0) return false;
        const uint64_t z = wave_at(B, 0);
        set_pos = comp_pos(z);
        ins_pos = set_pos;
        B = list_pop_front(B, nb);
        A = list_push_front(A, na, z, lane);
        clear_pos = xpos;
        B = list_insert<false>(B, nb, x, nb == out_before - 1, lane);
      }
    }
  }
  int ins_page = -1;
  if (phdr && ins_pos >= 0) {
    // a slot outside the kept records or a page outside the pools: rebuild instead
    if (ins_slot < 0 || ins_slot > kp || (ins_slot == kp && k == kp) || ins_slot >= p.pool.cap)
      return false;
    ins_page = ins_pos == xpos && xpage >= 0 ? xpage : pool_page(p.pool, b, ins_pos);
    if (ins_page < 0) return false;
  }
  if (lane == 0) {
    // the new position is protected (without protection it is the candidate,
    // cleared below if not kept); then the candidate changes
    __hip_atomic_fetch_or(&mrow[(L - 1) >> 5], 1u << ((L - 1) & 31), __ATOMIC_RELAXED,
                          __HIP_MEMORY_SCOPE_AGENT);
    if (set_pos >= 0)
      __hip_atomic_fetch_or(&mrow[set_pos >> 5], 1u << (set_pos & 31), __ATOMIC_RELAXED,
                            __HIP_MEMORY_SCOPE_AGENT);
    if (clear_pos >= 0)
      __hip_atomic_fetch_and(&mrow[clear_pos >> 5], ~(1u << (clear_pos & 31)), __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
    st->len = L;
    st->k = (int32_t)k;
    st->na = na;
    st->nb = nb;
  }
  if (lane < na) st->a[lane] = A;
  if (lane < nb) st->b[lane] = B;
  if (phdr) {
    if (ins_pos >= 0) {
      if (ins_pos == xpos && xpage >= 0) {  // the record fetched ahead
        if (lane < pool_chunks(p.pool.D))
          pool_put_chunk(pool_tile(p.pool, pair, ins_slot), p.pool.D, ins_slot % kPoolTile, lane, xrec);
      } else {
        pool_copy_wave(p.pool, pair, h, ins_page, ins_pos, ins_slot, lane);
      }
      if (lane == 0) {
        pool_slot_of(p.pool, pair)[ins_pos] = ins_slot;
        pool_pos_of(p.pool, pair)[ins_slot] = ins_pos;
      }
    }
    if (lane == 0) {
      phdr[0] = (int32_t)k;
      phdr[1] = L;
    }
  }
  return true;
}

// ---- kept-record pool in a full refresh. The mask pass compares each old
// mask word with the new one and lists, in position order, the kept INT4
// records that leave and those that enter; if the pool held exactly the old
// kept set and the lists fit, only those records move: entering records fill
// the slots of leaving ones (then extend the pool), and when the pool shrinks
// the records left in its tail move into the remaining holes below the new
// count. Otherwise the pool is rebuilt from the new mask (slots in position
// order).
constexpr int kDiffCap = 1024;  // changed records a refresh applies in place (one per thread)
static_assert(kDiffCap == kTopkThreads, "one changed record per thread");
struct PoolLds {
  int32_t rem[kDiffCap];   // positions leaving (position order); later the live tail slots
  int32_t add[kDiffCap];   // positions entering (position order)
  int32_t hole[kDiffCap];  // slot of rem[i]
  int32_t low[kDiffCap];   // holes below the new count, in rem order
  int32_t flag[kDiffCap];  // tail slot j (cnt_new + j) stays live
  uint32_t scan[kTopkThreads / 64];
  uint32_t oldpop;
};

// Block-wide exclusive prefix of one value per thread (in thread order).
__device__ inline uint32_t block_excl(uint32_t v, uint32_t* scan, uint32_t& total, int lane, int wid) {
  uint32_t incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t t = __shfl_up(incl, o);
    if (lane >= o) incl += t;
  }
  __syncthreads();
  if (lane == 63) scan[wid] = incl;
  __syncthreads();
  uint32_t base = 0;
  total = 0;
  for (int q = 0; q < kTopkThreads / 64; ++q) {
    const uint32_t x = scan[q];
    if (q < wid) base += x;
    total += x;
  }
  return base + incl - v;
}

// Bits of mask word w (positions 32w..32w+31) in [lo4, hi4).
__device__ inline uint32_t region_bits(int w, uint32_t word, int lo4, int hi4) {
  const int lo = lo4 - 32 * w, hi = hi4 - 32 * w;
  if (hi <= 0 || lo >= 32) return 0u;
  if (lo > 0) word &= ~0u << lo;
  if (hi < 32) word &= (1u << hi) - 1u;
  return word;
}

// The same, restricted to positions whose page is in the pools; pga / pgb
// receive the pages of the word's two halves.
__device__ inline uint32_t pool_word_bits(const PoolRef& r, int b, int w, uint32_t word, int lo4,
                                          int hi4, int& pga, int& pgb) {
  word = region_bits(w, word, lo4, hi4);
  if (word & 0x0000FFFFu) {
    pga = pool_page(r, b, 32 * w);
    if (pga < 0) word &= 0xFFFF0000u;
  }
  if (word & 0xFFFF0000u) {
    pgb = pool_page(r, b, 32 * w + 16);
    if (pgb < 0) word &= 0x0000FFFFu;
  }
  return word;
}

// Rebuild: every kept INT4 record of the new mask into slots 0, 1, ... in
// position order. Thread t reads back the words it wrote itself in the mask
// pass (same word-to-thread assignment), so no other thread's store is read.
// Returns the record count.
__device__ __attribute__((always_inline)) long long pool_rebuild(const TopkParams& p, PoolLds& ps, int pair, int b, int h, int n4,
                                  const uint32_t* mrow) {
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  int32_t* slot_of = pool_slot_of(p.pool, pair);
  int32_t* pos_of = pool_pos_of(p.pool, pair);
  long long pcarry = 0;
  for (int w0 = 0; w0 < p.words; w0 += kTopkThreads) {
    const int w = w0 + tid;
    int pga = -1, pgb = -1;
    uint32_t k4 = w < p.words ? pool_word_bits(p.pool, b, w, mrow[w], p.sink, p.sink + n4, pga, pgb) : 0u;
    uint32_t total;
    long long slot = pcarry + block_excl((uint32_t)__popc(k4), ps.scan, total, lane, wid);
    while (k4 != 0) {
      const int bit = __builtin_ctz(k4);
      k4 &= k4 - 1u;
      const int pos = 32 * w + bit;
      if (slot < p.pool.cap) {
        pool_copy_thread(p.pool, pair, h, bit < 16 ? pga : pgb, pos, (int)slot);
        slot_of[pos] = (int32_t)slot;
        pos_of[slot] = pos;
      }
      ++slot;
    }
    pcarry += total;
  }
  return pcarry;
}

// Applies nR leaving and nA entering records (lists in ps) to a pool of
// cnt_old records; returns the new count, or -1 (nothing changed) when the
// map does not place the leaving records in distinct slots below cnt_old.
__device__ __attribute__((always_inline)) int pool_apply(const TopkParams& p, PoolLds& ps, int pair, int b, int h, int cnt_old,
                          int nR, int nA) {
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  int32_t* slot_of = pool_slot_of(p.pool, pair);
  int32_t* pos_of = pool_pos_of(p.pool, pair);
  const int cnt_new = cnt_old - nR + nA;
  int hs = -1;
  if (tid < nR) {
    hs = slot_of[ps.rem[tid]];
    if (hs < 0 || hs >= cnt_old || pos_of[hs] != ps.rem[tid]) hs = -1;  // both maps must agree
    ps.hole[tid] = hs;
  }
  if (__syncthreads_or(tid < nR && hs < 0)) return -1;
  auto put = [&](int pos, int dst) {
    const int page = pool_page(p.pool, b, pos);
    if (page >= 0) pool_copy_thread(p.pool, pair, h, page, pos, dst);
    slot_of[pos] = dst;
    pos_of[dst] = pos;
  };
  if (nA >= nR) {
    if (tid < nA) put(ps.add[tid], tid < nR ? ps.hole[tid] : cnt_old + (tid - nR));
    return cnt_new;
  }
  // the pool shrinks: holes below cnt_new take the entering records, then the
  // records that stay live in the tail [cnt_new, cnt_old)
  const int tail = nR - nA;
  if (tid < tail) ps.flag[tid] = 1;
  __syncthreads();
  if (tid < nR && ps.hole[tid] >= cnt_new) ps.flag[ps.hole[tid] - cnt_new] = 0;
  __syncthreads();
  uint32_t nlow, nlive;
  const bool lowh = tid < nR && ps.hole[tid] < cnt_new;
  const uint32_t il = block_excl(lowh ? 1u : 0u, ps.scan, nlow, lane, wid);
  if (lowh) ps.low[il] = ps.hole[tid];
  const bool live = tid < tail && ps.flag[tid] != 0;
  const uint32_t iv = block_excl(live ? 1u : 0u, ps.scan, nlive, lane, wid);
  if (live) ps.rem[iv] = cnt_new + tid;
  __syncthreads();
  if (tid < (int)nlow) {
    const int dst = ps.low[tid];
    if (tid < nA) {
      put(ps.add[tid], dst);
    } else if (tid - nA < (int)nlive) {
      const int from = ps.rem[tid - nA];
      const int pos = pos_of[from];
      pool_move_thread(p.pool, pair, from, dst);
      if (pos >= 0 && pos < p.max_ctx) slot_of[pos] = dst;
      pos_of[dst] = pos;
    }
  }
  return cnt_new;
}

// ---- full refresh. An exact radix select over the 32-bit score keys (4
// passes of 8 bits, MSB first) finds, for up to three ranks at once, the key
// at that rank and how many keys equal to it lie within the rank: rank k
// (the threshold), and with a state to fill, ranks k - 63 and k + 64, which
// bound the keys the two lists must hold. The in-order mask pass keeps every
// key above the threshold and the lowest positions equal to it (the unique
// answer under "score descending, then position ascending"), and collects the
// keys between the two outer ranks; sorted, they give the lists.
// The full refresh of one (sequence, kv head) by the whole workgroup (the
// incremental step, when there is a state, has been tried by topk_group).
__device__ __attribute__((always_inline)) void topk_pair(const TopkParams& p, int h, int b) {
  __shared__ uint32_t hist[3][256];
  __shared__ uint32_t scan[kTopkThreads / 64];
  __shared__ uint32_t sel_digit[3], sel_above[3];
  __shared__ uint64_t cand[kCandCap];
  __shared__ uint32_t ncand;
  __shared__ PoolLds ps;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;
  int L = p.seq_lens[b];
  if (L < 0 || L > p.max_ctx) {
    if (tid == 0) report_error(p.pool.errors, KVC_ERR_LENGTH);
    L = L < 0 ? 0 : p.max_ctx;
  }
  const int n4 = L > p.sink + p.recent ? L - p.sink - p.recent : 0;
  const long long k = ((long long)p.budget * n4) / 1000;
  const float* sc = p.scores + ((size_t)b * p.hkv + h) * p.max_ctx + p.sink;
  uint32_t* mrow = p.mask + ((size_t)b * p.hkv + h) * p.words;
  TopkState* st = p.state ? p.state + (size_t)b * p.hkv + h : nullptr;

  if (tid == 0) {
    ncand = 0;
    ps.oldpop = 0;
  }
  __syncthreads();
  // a pool that holds exactly the kept records of an earlier length is
  // updated by the records that change; anything else is rebuilt
  const bool pooled = p.pool.cap > 0;
  const int pair = b * p.hkv + h;
  int len_old = -1, cnt_old = 0;
  if (pooled) {
    const int32_t* ph = p.pool.header + 4 * (size_t)pair;
    if ((uint32_t)ph[2] == kPoolMagic && ph[1] >= 0 && ph[1] <= p.max_ctx && ph[0] >= 0 &&
        ph[0] <= p.pool.cap) {
      len_old = ph[1];
      cnt_old = ph[0];
    }
  }
  const bool diff = len_old >= 0;
  const int n4_old = len_old > p.sink + p.recent ? len_old - p.sink - p.recent : 0;

  // ---- radix select: target 0 = rank k, 1 = rank k - 63, 2 = rank k + 64
  const bool all = k >= n4;
  long long rank[3];
  rank[0] = (k > 0 && !all) ? k : 0;
  rank[1] = (st && k > 0 && !all) ? (k - kTopkBuf + 1 > 1 ? k - kTopkBuf + 1 : 1) : 0;
  rank[2] = (st && k < n4) ? (k + kTopkBuf < n4 ? k + kTopkBuf : n4) : 0;
  uint32_t prefix[3] = {0, 0, 0};
  long long remaining[3] = {rank[0], rank[1], rank[2]};
  if (rank[0] > 0 || rank[1] > 0 || rank[2] > 0) {
    uint32_t pmask = 0;
    for (int pass = 0; pass < 4; ++pass) {
      const int shift = 24 - 8 * pass;
      // targets sharing a prefix share one histogram
      int src[3];
#pragma unroll
      for (int t = 0; t < 3; ++t) {
        src[t] = t;
        for (int u = 0; u < t; ++u)
          if (src[t] == t && rank[u] > 0 && prefix[u] == prefix[t]) src[t] = u;
      }
      for (int i = tid; i < 3 * 256; i += kTopkThreads) hist[i >> 8][i & 255] = 0;
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
            const uint32_t dg = (key >> shift) & 255u;
#pragma unroll
            for (int t = 0; t < 3; ++t)
              if (rank[t] > 0 && src[t] == t && (key & pmask) == prefix[t]) atomicAdd(&hist[t][dg], 1u);
          }
        }
      }
      __syncthreads();
      if (wid < 3 && rank[wid] > 0) {
        // lane l owns bins 4l..4l+3 of the target's histogram; suffix sums from the top bin down
        const uint32_t* hh = hist[src[wid]];
        const long long want = remaining[wid];
        uint32_t c0 = hh[4 * lane], c1 = hh[4 * lane + 1], c2 = hh[4 * lane + 2], c3 = hh[4 * lane + 3];
        const uint32_t s4 = c0 + c1 + c2 + c3;
        uint32_t suf = s4;  // inclusive suffix over lanes >= lane
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          const uint32_t t = __shfl_down(suf, o);
          if (lane + o < 64) suf += t;
        }
        const uint32_t above = suf - s4;  // keys in bins of higher lanes
        if ((long long)above < want && want <= (long long)suf) {
          uint32_t acc = above;
          int d = 4 * lane + 3;
          const uint32_t cs[4] = {c0, c1, c2, c3};
          for (int q = 3; q >= 0; --q) {
            if ((long long)(acc + cs[q]) >= want) { d = 4 * lane + q; break; }
            acc += cs[q];
          }
          sel_digit[wid] = (uint32_t)d;
          sel_above[wid] = acc;
        }
      }
      __syncthreads();
#pragma unroll
      for (int t = 0; t < 3; ++t) {
        if (rank[t] > 0) {
          remaining[t] -= sel_above[t];
          prefix[t] |= sel_digit[t] << shift;
        }
      }
      pmask |= 255u << shift;
      __syncthreads();
    }
  }
  // threshold: keys > T kept, and the first `need` keys == T (in position order)
  const uint32_t T = rank[0] > 0 ? prefix[0] : 0xFFFFFFFFu;
  const long long need = rank[0] > 0 ? remaining[0] : 0;
  // window of keys the lists need, and how many keys lie above it
  const uint32_t hi = rank[1] > 0 ? prefix[1] : 0xFFFFFFFFu;
  const uint32_t lo = rank[2] > 0 ? prefix[2] : 0u;
  const long long above_hi = rank[1] > 0 ? rank[1] - remaining[1] : 0;

  // ---- in-order pass: one mask word per thread, block-wide running count of
  // keys == T. With a pool in diff mode, the records leaving and entering are
  // listed in position order (rcarry / acarry count them so far).
  long long carry = 0;
  long long rcarry = 0, acarry = 0;
  uint32_t oldpop = 0;
  for (int w0 = 0; w0 < p.words; w0 += kTopkThreads) {
    const int w = w0 + tid;
    uint32_t gt = 0, eq = 0;  // bit masks over the word's INT4 positions
    if (w < p.words && n4 > 0 && (st || (k > 0 && !all))) {
      float v[32];
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        const int t = w * 32 + i;
        v[i] = (t >= p.sink && t < p.sink + n4) ? sc[t - p.sink] : 0.0f;
      }
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        const int t = w * 32 + i;
        if (t >= p.sink && t < p.sink + n4) {
          const uint32_t key = order_key(v[i]);
          if (key > T) gt |= 1u << i;
          else if (key == T) eq |= 1u << i;
          if (st && !all && key >= lo && key <= hi) {
            const uint32_t slot = atomicAdd(&ncand, 1u);
            if (slot < kCandCap) cand[slot] = comp_key(key, t);
          }
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
    uint32_t wbits = 0, oldw = 0;  // the word as written, and as it was
    if (w < p.words) {
      if (pooled && diff) oldw = mrow[w];
      uint32_t bits = (k > 0 && !all) ? gt : 0u;
      if (eq && k > 0 && !all) {
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
        const bool prot = t < p.sink || (p.recent > 0 && t >= L - p.recent);
        if (prot || (all && t >= p.sink)) bits |= 1u << i;
      }
      mrow[w] = bits;
      wbits = bits;
    }
    carry += tile_total;
    if (pooled && diff) {
      uint32_t remw = 0, addw = 0;
      if (w < p.words) {
        int pa = -1, pb = -1;
        // the old records are not read, so their pages are not looked up
        const uint32_t old_in = region_bits(w, oldw, p.sink, p.sink + n4_old);
        const uint32_t new_in = pool_word_bits(p.pool, b, w, wbits, p.sink, p.sink + n4, pa, pb);
        oldpop += (uint32_t)__popc(old_in);
        remw = old_in & ~new_in;
        addw = new_in & ~old_in;
      }
      uint32_t both;
      const uint32_t ex = block_excl((uint32_t)__popc(remw) | ((uint32_t)__popc(addw) << 16), ps.scan,
                                     both, lane, wid);
      long long ir = rcarry + (ex & 0xFFFFu), ia = acarry + (ex >> 16);
      for (; remw; remw &= remw - 1u, ++ir)
        if (ir < kDiffCap) ps.rem[ir] = 32 * w + __builtin_ctz(remw);
      for (; addw; addw &= addw - 1u, ++ia)
        if (ia < kDiffCap) ps.add[ia] = 32 * w + __builtin_ctz(addw);
      rcarry += both & 0xFFFFu;
      acarry += both >> 16;
    }
    __syncthreads();
  }
  if (pooled) {
    if (diff) atomicAdd(&ps.oldpop, oldpop);
    __syncthreads();
    const long long cnt_new = (long long)cnt_old - rcarry + acarry;
    long long count = -1;
    if (diff && rcarry <= kDiffCap && acarry <= kDiffCap && ps.oldpop == (uint32_t)cnt_old &&
        cnt_new <= p.pool.cap)
      count = pool_apply(p, ps, pair, b, h, cnt_old, (int)rcarry, (int)acarry);
    if (count < 0) count = pool_rebuild(p, ps, pair, b, h, n4, mrow);
    __syncthreads();
    if (tid == 0) {
      int32_t* phdr = p.pool.header + 4 * (size_t)pair;
      const bool fits = count <= p.pool.cap;
      if (!fits) report_error(p.pool.errors, KVC_ERR_POOL);
      phdr[0] = (int32_t)(fits ? count : p.pool.cap);
      phdr[1] = L;
      phdr[2] = fits ? (int32_t)kPoolMagic : 0;
      phdr[3] = 0;
    }
  }
  if (!st) return;

  // ---- lists: sort the window (descending composite keys) and cut at rank k
  const uint32_t nc = ncand;
  const bool fits = nc <= kCandCap;
  if (fits) {
    int n2 = 1;
    while (n2 < (int)nc) n2 <<= 1;
    for (int i = tid; i < n2; i += kTopkThreads)
      if (i >= (int)nc) cand[i] = 0;  // below every real key (positions < 2^32 - 1)
    __syncthreads();
    for (int size = 2; size <= n2; size <<= 1) {
      for (int stride = size >> 1; stride > 0; stride >>= 1) {
        for (int i = tid; i < n2; i += kTopkThreads) {
          const int j = i ^ stride;
          if (j > i) {
            const bool desc = (i & size) == 0;
            const uint64_t x = cand[i], y = cand[j];
            if (desc ? x < y : x > y) { cand[i] = y; cand[j] = x; }
          }
        }
        __syncthreads();
      }
    }
  }
  // global rank (1-based) of cand[i] is above_hi + i + 1
  // with every position kept the lists stay empty (the in-place update never
  // consults them while the budget stays 1000)
  const int na = all ? 0 : (int)(k < kTopkBuf ? k : kTopkBuf);
  const int nb = all ? 0 : (int)(n4 - k < kTopkBuf ? n4 - k : kTopkBuf);
  if (wid == 0) {
    bool ok = fits || all;
    if (ok && lane < na) {
      const long long i = k - lane - above_hi - 1;
      if (i >= 0 && i < nc) st->a[lane] = cand[i];
      else ok = false;
    }
    if (ok && lane < nb) {
      const long long i = k + lane - above_hi;
      if (i >= 0 && i < nc) st->b[lane] = cand[i];
      else ok = false;
    }
    ok = __ballot(!ok) == 0;
    if (lane == 0) {
      st->len = L;
      st->k = (int32_t)k;
      st->budget = p.budget;
      st->na = na;
      st->nb = nb;
      st->magic = ok ? kTopkMagic : 0u;
    }
  }
}

// ---- block-granular refresh (KVP promo page, "Engineering limits": a paged
// cache evicts whole blocks, ranked by the mean score of their tokens, after an
// optional coarse recency cut). Region offsets o = position - 16; block j of
// B tokens covers offsets [Bj, Bj + B); offsets below c0 (the recency cut) are
// not candidates. A block's key is the order key of the float32 mean of its
// candidate scores, summed in position order. One workgroup per (sequence,
// kv head).
struct BlockTopkParams {
  const float* scores;
  const int32_t* seq_lens;
  uint32_t* mask;
  unsigned char* state;  // per-pair BlockStateHeader + keys, or NULL
  size_t state_stride;   // bytes per (sequence, kv head)
  int hkv;
  int max_ctx;
  int words;
  int budget;
  int window;
  int sink, recent;  // INT8-protected sink and recent positions (16/128, or 0/0)
  PoolRef pool;      // kept-record pool maintained with the mask (pool.cap = 0: none)
};

constexpr int kBlockWaves = kTopkThreads / 64;
constexpr int kBlockKeysLds = 32768;  // block keys cached in LDS up to this many blocks
constexpr int kBlockBitWords = kMaxBlocks / 32;  // kept-block bitmap
constexpr int kChunkPos = 256;        // offsets one wave loads per 16-byte load (4 per lane)
constexpr int kRoundChunks = 8;       // loads a wave keeps in flight per round

struct BlockLds {
  uint32_t keys[kBlockKeysLds];
  uint32_t kept_bits[kBlockBitWords];
  uint32_t seg[kMaxBlocks / 64];  // per 64-block segment: keys equal to T, then their prefix
  uint32_t hist[256];
  uint32_t red[2][kBlockWaves];
  uint32_t sel_digit, sel_above, sel_count;
};

// Four consecutive scores; p is 16-byte aligned when vec is set.
__device__ inline float4 load_scores4(const float* p, bool vec) {
  if (vec) return *reinterpret_cast<const float4*>(p);
  return make_float4(p[0], p[1], p[2], p[3]);
}

// Histogram add of one digit per active lane; lanes of a wave sharing a digit
// are added together (a few rounds), the rest one by one.
__device__ inline void hist_add(uint32_t* hist, uint32_t d, bool active, int lane) {
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const uint64_t am = __ballot(active);
    if (am == 0) return;
    const int first = __ffsll((long long)am) - 1;
    const uint32_t d0 = __shfl(d, first);
    const uint64_t same = __ballot(active && d == d0);
    if (lane == first) atomicAdd(&hist[d0], (uint32_t)__popcll(same));
    if (d == d0) active = false;
  }
  if (active) atomicAdd(&hist[d], 1u);
}

// Workgroup sums of two counters (every thread gets both totals).
__device__ inline void block_sum2(BlockLds& sm, uint32_t& x, uint32_t& y, int lane, int wid) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    x += __shfl_xor(x, o);
    y += __shfl_xor(y, o);
  }
  if (lane == 0) {
    sm.red[0][wid] = x;
    sm.red[1][wid] = y;
  }
  __syncthreads();
  x = 0;
  y = 0;
  for (int q = 0; q < kBlockWaves; ++q) {
    x += sm.red[0][q];
    y += sm.red[1][q];
  }
  __syncthreads();
}

// The smallest key above t (up) or the largest key below t (!up) among n
// keys, with its multiplicity (cnt = 0 when there is none); workgroup-wide.
template <typename KeyOf>
__device__ inline void block_next_key(BlockLds& sm, KeyOf key_of, int n, uint32_t t, bool up,
                                      uint32_t& best, uint32_t& cnt, int tid, int lane, int wid) {
  best = 0;
  cnt = 0;
  auto merge = [&](uint32_t k, uint32_t c) {
    if (c == 0) return;
    if (cnt == 0 || (up ? k < best : k > best)) {
      best = k;
      cnt = c;
    } else if (k == best) {
      cnt += c;
    }
  };
#pragma unroll 4
  for (int i = tid; i < n; i += kTopkThreads) {
    const uint32_t k = key_of(i);
    if (up ? k > t : k < t) merge(k, 1);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const uint32_t ob = __shfl_xor(best, o);
    const uint32_t oc = __shfl_xor(cnt, o);
    merge(ob, oc);
  }
  if (lane == 0) {
    sm.red[0][wid] = best;
    sm.red[1][wid] = cnt;
  }
  __syncthreads();
  best = 0;
  cnt = 0;
  for (int q = 0; q < kBlockWaves; ++q) merge(sm.red[0][q], sm.red[1][q]);
  __syncthreads();
}

// Bits of positions [lo, hi) that fall in the mask word starting at position base.
__device__ inline uint32_t range_bits(int lo, int hi, int base) {
  lo -= base;
  hi -= base;
  if (lo < 0) lo = 0;
  if (hi > 32) hi = 32;
  if (hi <= lo) return 0u;
  const uint32_t upto_hi = hi == 32 ? 0xFFFFFFFFu : ((1u << hi) - 1u);
  return upto_hi & ~((1u << lo) - 1u);
}

// Key of block j from its candidate scores, one load at a time (for the rare
// stateless refresh of more blocks than LDS caches).
template <int B>
__device__ inline uint32_t block_key_serial(const float* sc, int j, int c0, int n4) {
  const int a = B * j > c0 ? B * j : c0;
  const int e = B * j + B < n4 ? B * j + B : n4;
  float sum = 0.0f;
  for (int t = a; t < e; ++t) sum += sc[t];
  return order_key(sum / (float)(e - a));
}

// Key of block j from its candidate scores, loaded up to 32 at a time.
template <int B>
__device__ inline uint32_t block_key_direct(const float* sc, int j, int c0, int n4) {
  constexpr int kPart = B < 32 ? B : 32;
  const int a = B * j > c0 ? B * j : c0;
  const int e = B * j + B < n4 ? B * j + B : n4;
  float sum = 0.0f;
#pragma unroll
  for (int c = 0; c < B; c += kPart) {
    float v[kPart];
#pragma unroll
    for (int i = 0; i < kPart; ++i) v[i] = a + c + i < e ? sc[a + c + i] : 0.0f;
#pragma unroll
    for (int i = 0; i < kPart; ++i)
      if (a + c + i < e) sum += v[i];
  }
  return order_key(sum / (float)(e - a));
}

// Mask word w (positions 32w..32w+31) of a sequence of length L: protected
// positions [0, min(L, sink)) and [rec0, L) set, candidates [lo4, hi4) set
// where their block is kept; a word meets at most two blocks, jA and jB.
template <int B, typename Kept>
__device__ inline uint32_t block_mask_word(int w, int L, int sink, int rec0, int lo4, int hi4,
                                           Kept kept_block) {
  const int base = 32 * w;
  uint32_t bits = range_bits(0, L < sink ? L : sink, base) | range_bits(rec0, L, base);
  const uint32_t cand = range_bits(lo4, hi4, base);
  if (cand) {
    const int jA = (base - sink + B) / B - 1;  // floor((base - sink) / B), base - sink >= -B
    const int jB = (base + 31 - sink) / B;
    const int split = sink + B * jB;
    uint32_t kb = 0;
    if (kept_block(jA)) kb |= range_bits(sink + B * jA, split, base);
    if (kept_block(jB)) kb |= range_bits(split, split + B, base);
    bits |= cand & kb;
  }
  return bits;
}

// The refresh of p.group pairs in one workgroup (1, or up to kTopkGroup in a
// decode step with a state): wave w applies the incremental step (topk_step,
// one wave's work) to pair p.group * g + w, so that a step over thousands of
// pairs is one resident round of workgroups instead of several rounds of one
// 1024-thread workgroup per pair; the pairs whose step does not apply (no
// state, a list ran out, a new budget, a stale state) are then refreshed in
// full one after another by the whole workgroup (topk_pair). Each pair gets
// the same result whatever the grouping.
__device__ __attribute__((always_inline)) void topk_group(const TopkParams& p, int g) {
  __shared__ uint32_t need;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;
  if (tid == 0) need = 0;
  __syncthreads();
  const int pair = g * p.group + wid;
  if (wid < p.group && pair < p.pairs) {
    const int b = pair / p.hkv, h = pair % p.hkv;
    int L = p.seq_lens[b];
    bool ok = false;
    if (L >= 0 && L <= p.max_ctx && p.state && p.incremental) {
      const int n4 = L > p.sink + p.recent ? L - p.sink - p.recent : 0;
      const long long k = ((long long)p.budget * n4) / 1000;
      const float* sc = p.scores + ((size_t)b * p.hkv + h) * p.max_ctx + p.sink;
      uint32_t* mrow = p.mask + ((size_t)b * p.hkv + h) * p.words;
      ok = topk_step(p, p.state + (size_t)b * p.hkv + h, L, n4, k, sc, mrow, lane, b, h);
    }
    if (!ok && lane == 0) atomicOr(&need, 1u << wid);
  }
  __syncthreads();
  uint32_t nd = need;
  while (nd) {
    const int w = __builtin_ctz(nd);
    nd &= nd - 1;
    const int q = g * p.group + w;
    topk_pair(p, q % p.hkv, q / p.hkv);
    __syncthreads();
  }
}


// POOL: the kept-record pool is maintained with the mask (a separate
// instance, so that the kernels without a pool keep their own code).
template <int B, bool POOL>
__device__ void block_topk_pair(const BlockTopkParams& p, BlockLds& sm, int h, int b) {
  static_assert(B == 16 || B == 32 || B == 64, "block size");
  constexpr int kOldWords = 5;  // previous mask words held per thread (the rest re-read)
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  int L = p.seq_lens[b];
  if (L < 0) L = 0;
  if (L > p.max_ctx) L = p.max_ctx;
  const int sink = p.sink, slots = p.sink + p.recent;
  const int n4 = L > slots ? L - slots : 0;
  const int c0 = p.window > 0 ? (n4 - p.window > 0 ? n4 - p.window : 0) : 0;
  const int j0 = c0 / B;
  const int nb = n4 > c0 ? (n4 + B - 1) / B - j0 : 0;
  const long long k = ((long long)p.budget * nb) / 1000;
  const bool all = k >= nb;
  const bool select = k > 0 && !all;
  const float* sc = p.scores + ((size_t)b * p.hkv + h) * p.max_ctx + sink;
  uint32_t* mrow = p.mask + ((size_t)b * p.hkv + h) * p.words;
  const bool cached = nb <= kBlockKeysLds;
  BlockStateHeader* st = p.state ? reinterpret_cast<BlockStateHeader*>(
                                       p.state + ((size_t)b * p.hkv + h) * p.state_stride)
                                 : nullptr;
  uint32_t* skeys = st ? reinterpret_cast<uint32_t*>(st + 1) : nullptr;
  // keys are stored (LDS cache, state) only where something keeps them
  const bool need_keys = (select && cached) || st != nullptr;

  bool valid = false, thr_ok = false;
  int len0 = 0;
  uint32_t thr0 = 0;
  if (st) {
    const uint32_t magic = st->magic;
    len0 = st->len;
    valid = magic == kBlockMagic && st->block == B && st->window == p.window && len0 >= 0 &&
            len0 <= L;
    thr_ok = valid && st->has_thr != 0 && st->budget == p.budget;
    thr0 = st->thr;
  }
  // a pool that holds exactly the kept records of an earlier length is updated
  // by the records that change (as in the token refresh); anything else, and
  // masks longer than the words a thread keeps, is rebuilt
  // The pool's header is loaded here with the state but not looked at before
  // the key passes, so that it adds no round trip of its own.
  const bool pooled = POOL && p.pool.cap > 0;
  const int pair = b * p.hkv + h;
  int32_t ph0 = 0, ph1 = -1, ph2 = 0;
  if (pooled) {
    const int32_t* ph = p.pool.header + 4 * (size_t)pair;
    ph0 = ph[0];
    ph1 = ph[1];
    ph2 = ph[2];
  }
  // keys above / equal to thr0 as the state left them, and which old keys leave
  const int n4o = len0 > slots ? len0 - slots : 0;
  const int c0o = p.window > 0 ? (n4o - p.window > 0 ? n4o - p.window : 0) : 0;
  const int j0o = c0o / B;
  const int nbo = n4o > c0o ? (n4o + B - 1) / B - j0o : 0;
  const int nrem = j0 > j0o ? j0 - j0o : 0;  // blocks the moved cut removed: [j0o, j0)
  uint32_t gt_st = 0, eq_st = 0;
  bool counted = false;
  if (thr_ok && select && cached && st->has_cnt != 0 && nrem <= kTopkThreads) {
    gt_st = st->gt;
    eq_st = st->eq;
    counted = true;
  }

  // ---- everything the full refresh reads is loaded up front: the previous
  // mask words, the state's keys (into LDS), and the keys of the first and the
  // last candidate block (the ones a one-token step changes)
  uint32_t old_w[kOldWords];
#pragma unroll
  for (int m = 0; m < kOldWords; ++m) {
    const int w = tid + m * kTopkThreads;
    old_w[m] = w < p.words ? mrow[w] : 0u;
  }
  int spec_r = -1;
  uint32_t spec_key = 0;
  if (need_keys && nb > 0) {
    if (tid == kTopkThreads - 1) spec_r = nb - 1;
    if (tid == kTopkThreads - 2 && nb > 1) spec_r = 0;
    if (spec_r >= 0) spec_key = block_key_direct<B>(sc, j0 + spec_r, c0, n4);
  }
  if (st && cached) {
#pragma unroll 8
    for (int i = tid; i < nb; i += kTopkThreads) sm.keys[i] = skeys[j0 + i];
  }
  // counted: the counts against thr0 follow from the keys that change (the
  // removed ones, loaded here, and the recomputed ones below), not a full pass
  int dgt = 0, deq = 0;
  if (counted && tid < nrem && tid < nbo) {
    const uint32_t old = skeys[j0o + tid];
    dgt -= old > thr0;
    deq -= old == thr0;
  }
  // the previous mask words are needed only at the end; keep them here, with
  // this round of loads, instead of a round trip of their own later
#pragma unroll
  for (int m = 0; m < kOldWords; ++m) asm volatile("" ::"v"(old_w[m]));

  // keys recomputed from the scores: relative blocks [ra, nb), and block 0
  // when the recency cut moved (blocks in between are full and unchanged)
  int ra = 0;
  bool first_too = false;
  if (valid) {
    ra = n4o / B - j0;
    if (ra < 0) ra = 0;
    if (ra > nb) ra = nb;
    first_too = c0o != c0 && ra > 0;
  }
  __syncthreads();  // header read and state keys in LDS before anything is rewritten

  auto store_key = [&](int r, uint32_t key) {
    if (counted) {  // each recomputed block is stored by exactly one thread
      const int a = j0 + r;
      if (a >= j0o && a < j0o + nbo) {
        const uint32_t old = sm.keys[r];
        dgt -= old > thr0;
        deq -= old == thr0;
      }
      dgt += key > thr0;
      deq += key == thr0;
    }
    if (cached) sm.keys[r] = key;
    if (st) skeys[j0 + r] = key;
  };
  if (need_keys && nb - ra >= kTopkThreads) {
    // many keys: a wave round covers kRoundChunks * 256 consecutive offsets,
    // lane l holding offsets 4l..4l+3 of each 256; the B/4 lanes of one block
    // pass the running sum along in position order
    constexpr int kLanesPerBlock = B / 4;
    constexpr int kChunks = B == 64 ? kRoundChunks / 2 : kRoundChunks;  // longer chains, fewer loads
    constexpr int kBlocksPerChunk = kChunkPos / B;
    constexpr int kBlocksPerRound = kChunks * kBlocksPerChunk;
    const bool vec = (reinterpret_cast<uintptr_t>(sc) & 15) == 0;
    const int sub = lane % kLanesPerBlock;
    for (int g = wid; ra + g * kBlocksPerRound < nb; g += kBlockWaves) {
      const int ob = B * (j0 + ra + g * kBlocksPerRound) + 4 * lane;
      float4 v[kChunks];
#pragma unroll
      for (int u = 0; u < kChunks; ++u) {
        const int o = ob + u * kChunkPos;
        v[u] = o < n4 ? load_scores4(sc + o, vec) : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
      }
#pragma unroll
      for (int u = 0; u < kChunks; ++u) {
        const int r = ra + g * kBlocksPerRound + u * kBlocksPerChunk + lane / kLanesPerBlock;
        const int j = j0 + r;
        const int a = B * j > c0 ? B * j : c0;
        const int e = B * j + B < n4 ? B * j + B : n4;
        const int o = ob + u * kChunkPos;
        float run = 0.0f;
#pragma unroll
        for (int t = 0; t < kLanesPerBlock; ++t) {
          const float prev = __shfl_up(run, 1, kLanesPerBlock);
          if (sub == t) {
            float x = t == 0 ? 0.0f : prev;
            if (o >= a && o < e) x += v[u].x;
            if (o + 1 >= a && o + 1 < e) x += v[u].y;
            if (o + 2 >= a && o + 2 < e) x += v[u].z;
            if (o + 3 >= a && o + 3 < e) x += v[u].w;
            run = x;
          }
        }
        if (sub == kLanesPerBlock - 1 && r < nb) store_key(r, order_key(run / (float)(e - a)));
      }
    }
    if (first_too && spec_r == 0) store_key(0, spec_key);
  } else if (need_keys) {
    // few keys: one block per thread; the first and the last block come from
    // the threads that computed them up front
    if (spec_r >= 0 && (spec_r >= ra || (spec_r == 0 && first_too))) store_key(spec_r, spec_key);
    const int r = ra + tid;
    if (r < nb && r != nb - 1 && !(r == 0 && nb > 1)) store_key(r, block_key_direct<B>(sc, j0 + r, c0, n4));
  }
  __syncthreads();
  auto key_of = [&](int i) -> uint32_t {
    if (cached) return sm.keys[i];
    if (st) return skeys[j0 + i];
    return block_key_serial<B>(sc, j0 + i, c0, n4);
  };

  // ---- threshold T = key of the k-th largest block; need = blocks with key T
  // kept (lowest block first) out of eqT with that key
  uint32_t T = 0u;
  long long need = 0, eqT = 0;
  if (select) {
    bool found = false;
    if (thr_ok) {
      // start from the previous threshold: count the keys above and equal to
      // it, then move it to the next distinct key up or down while it selects
      // more or fewer than k blocks (a few keys change from call to call)
      uint32_t gt = 0, eq = 0;
      if (counted) {
        gt = (uint32_t)dgt;
        eq = (uint32_t)deq;
        block_sum2(sm, gt, eq, lane, wid);
        gt += gt_st;
        eq += eq_st;
      } else {
#pragma unroll 8
        for (int i = tid; i < nb; i += kTopkThreads) {
          const uint32_t key = key_of(i);
          gt += key > thr0;
          eq += key == thr0;
        }
        block_sum2(sm, gt, eq, lane, wid);
      }
      uint32_t t = thr0;
      for (int step = 0; step < 4; ++step) {
        if ((long long)gt < k && k <= (long long)gt + eq) {
          T = t;
          need = k - gt;
          eqT = eq;
          found = true;
          break;
        }
        if (step == 3) break;
        const bool up = (long long)gt >= k;
        uint32_t nt, nc;
        block_next_key(sm, key_of, nb, t, up, nt, nc, tid, lane, wid);
        if (nc == 0) break;
        if (up) {
          gt -= nc;
        } else {
          gt += eq;
        }
        t = nt;
        eq = nc;
      }
    }
    if (!found) {  // radix select, 8 bits per pass
      uint32_t prefix = 0, pmask = 0;
      long long remaining = k;
      for (int pass = 0; pass < 4; ++pass) {
        const int shift = 24 - 8 * pass;
        for (int i = tid; i < 256; i += kTopkThreads) sm.hist[i] = 0;
        __syncthreads();
        for (int i0 = 0; i0 < nb; i0 += kTopkThreads) {
          const int i = i0 + tid;
          const uint32_t key = i < nb ? key_of(i) : 0u;
          hist_add(sm.hist, (key >> shift) & 255u, i < nb && (key & pmask) == prefix, lane);
        }
        __syncthreads();
        if (wid == 0) {
          uint32_t c4[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) c4[q] = sm.hist[4 * lane + q];
          const uint32_t s4 = c4[0] + c4[1] + c4[2] + c4[3];
          uint32_t suf = s4;  // keys whose digit is >= 4 * lane
#pragma unroll
          for (int o = 1; o < 64; o <<= 1) {
            const uint32_t t = __shfl_down(suf, o);
            if (lane + o < 64) suf += t;
          }
          const uint32_t above = suf - s4;
          if ((long long)above < remaining && remaining <= (long long)suf) {
            uint32_t acc = above;
            int d = 4 * lane, cd = c4[0];
            for (int q = 3; q >= 0; --q) {
              if ((long long)(acc + c4[q]) >= remaining) {
                d = 4 * lane + q;
                cd = c4[q];
                break;
              }
              acc += c4[q];
            }
            sm.sel_digit = (uint32_t)d;
            sm.sel_above = acc;
            sm.sel_count = (uint32_t)cd;
          }
        }
        __syncthreads();
        remaining -= sm.sel_above;
        prefix |= sm.sel_digit << shift;
        pmask |= 255u << shift;
        eqT = sm.sel_count;  // after the last pass: keys equal to the threshold
        __syncthreads();
      }
      T = prefix;
      need = remaining;
    }
  }
  // with every tie at T kept (always so for distinct keys), kept = key >= T
  const bool by_key = select && need == eqT;

  // ---- otherwise a kept flag per candidate block, by 64-block segments (wave
  // ballots): ties at T are kept in block order, ranked by a segment prefix
  if (select && !by_key) {
    const int nseg = (nb + 63) / 64;
    const uint64_t below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
    for (int sg = wid; sg < nseg; sg += kBlockWaves) {
      const int i = 64 * sg + lane;
      const uint64_t eqs = __ballot(i < nb && key_of(i) == T);
      if (lane == 0) sm.seg[sg] = (uint32_t)__popcll(eqs);
    }
    __syncthreads();
    if (wid == 0) {  // exclusive prefix of the segment counts
      const int per = (nseg + 63) / 64;
      const int lo = lane * per < nseg ? lane * per : nseg;
      const int hi = lo + per < nseg ? lo + per : nseg;
      uint32_t sum = 0;
      for (int q = lo; q < hi; ++q) sum += sm.seg[q];
      uint32_t incl = sum;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const uint32_t t = __shfl_up(incl, o);
        if (lane >= o) incl += t;
      }
      uint32_t run = incl - sum;
      for (int q = lo; q < hi; ++q) {
        const uint32_t c = sm.seg[q];
        sm.seg[q] = run;
        run += c;
      }
    }
    __syncthreads();
    for (int sg = wid; sg < nseg; sg += kBlockWaves) {
      const int i = 64 * sg + lane;
      bool kept = false, eq = false;
      if (i < nb) {
        const uint32_t key = key_of(i);
        kept = key > T;
        eq = key == T;
      }
      const uint64_t eqs = __ballot(eq);
      if (eq) kept = (long long)sm.seg[sg] + __popcll(eqs & below) < need;
      const uint64_t ks = __ballot(kept);
      if (lane == 0) sm.kept_bits[2 * sg] = (uint32_t)ks;
      if (lane == 32) sm.kept_bits[2 * sg + 1] = (uint32_t)(ks >> 32);
    }
    __syncthreads();
  }

  // ---- kept-block bitmap when kept means key >= T and the keys are not in
  // LDS: one ballot per 64-block segment (the tie case filled it above; with
  // every block kept, or the keys in LDS, the words test the keys directly)
  const bool direct = all || (by_key && cached);
  if (by_key && !cached) {
    const int nseg = (nb + 63) / 64;
    for (int sg = wid; sg < nseg; sg += kBlockWaves) {
      const int i = 64 * sg + lane;
      const uint64_t ks = __ballot(i < nb && key_of(i) >= T);
      if (lane == 0) sm.kept_bits[2 * sg] = (uint32_t)ks;
      if (lane == 32) sm.kept_bits[2 * sg + 1] = (uint32_t)(ks >> 32);
    }
    __syncthreads();
  }

  // ---- mask words: protected positions kept, kept blocks' candidates kept,
  // everything else (evicted, cut, positions >= L) clear; a word is stored only
  // where it differs from what the mask holds. Word w (positions 32w..32w+31)
  // meets at most two blocks, jA and jB, jB starting at position split.
  // protected: [0, min(L, sink)) and [max(sink, L - recent), L) (none without protection)
  const int rec0 = p.recent == 0 ? L : (L - p.recent > sink ? L - p.recent : sink);
  const int lo4 = sink + c0, hi4 = sink + n4;
  const bool any_kept = all || select;
  auto kept_block = [&](int j) -> bool {
    const int r = j - j0;
    if (!any_kept || r < 0 || r >= nb) return false;
    if (direct) return all || sm.keys[r] >= T;
    return ((sm.kept_bits[r >> 5] >> (r & 31)) & 1u) != 0;
  };
  auto word_bits = [&](int w) -> uint32_t {
    return block_mask_word<B>(w, L, sink, rec0, lo4, hi4, kept_block);
  };
  // a pool that holds exactly the kept records of an earlier length is updated
  // by the records that change (as in the token refresh); anything else, and
  // masks longer than the words a thread keeps, is rebuilt
  int plen_old = -1, pcnt_old = 0;
  if ((uint32_t)ph2 == kPoolMagic && ph1 >= 0 && ph1 <= p.max_ctx && ph0 >= 0 && ph0 <= p.pool.cap) {
    plen_old = ph1;
    pcnt_old = ph0;
  }
  const bool pdiff = pooled && plen_old >= 0 && p.words <= kOldWords * kTopkThreads;
  const int pn4_old = plen_old > slots ? plen_old - slots : 0;
  // pool: per word, the kept INT4 records that leave and those that enter
  uint32_t remw[POOL ? kOldWords : 1], addw[POOL ? kOldWords : 1], oldpop = 0;
#pragma unroll
  for (int m = 0; m < kOldWords; ++m) {
    const int w = tid + m * kTopkThreads;
    if constexpr (POOL) remw[m] = addw[m] = 0u;
    if (w < p.words) {
      const uint32_t bits = word_bits(w);
      if (bits != old_w[m]) mrow[w] = bits;
      if constexpr (POOL) if (pdiff) {
        // only entering records have their pages looked up (a record the pool
        // holds stays valid while the caller keeps the table, as the pool
        // contract requires), so a word without one costs no load
        const uint32_t old_in = region_bits(w, old_w[m], sink, sink + pn4_old);
        const uint32_t new_in = region_bits(w, bits, sink, sink + n4);
        oldpop += (uint32_t)__popc(old_in);
        remw[m] = old_in & ~new_in;
        uint32_t add = new_in & ~old_in;
        if (add) {
          int pa = -1, pb = -1;
          add = pool_word_bits(p.pool, b, w, add, sink, sink + n4, pa, pb);
        }
        addw[m] = add;
      }
    }
  }
  for (int w = tid + kOldWords * kTopkThreads; w < p.words; w += kTopkThreads) {
    const uint32_t bits = word_bits(w);
    if (bits != mrow[w]) mrow[w] = bits;
  }
  if constexpr (POOL) if (pooled) {
    // the keys and the kept-block bitmap are no longer read: their LDS holds
    // the pool's lists
    static_assert(sizeof(PoolLds) <= sizeof(sm.keys), "pool lists fit the key cache");
    PoolLds& ps = *reinterpret_cast<PoolLds*>(sm.keys);
    uint32_t mine = 0;
#pragma unroll
    for (int m = 0; m < kOldWords; ++m) mine |= remw[m] | addw[m];
    // (the barrier also ends every read of the keys, whose LDS ps reuses)
    const bool changes = __syncthreads_or(mine != 0) != 0;
    if (tid == 0) ps.oldpop = 0;
    __syncthreads();
    long long rcarry = 0, acarry = 0;
#pragma unroll
    for (int m = 0; m < kOldWords && changes; ++m) {
      const int w = tid + m * kTopkThreads;
      uint32_t both;
      const uint32_t ex = block_excl((uint32_t)__popc(remw[m]) | ((uint32_t)__popc(addw[m]) << 16),
                                     ps.scan, both, lane, wid);
      long long ir = rcarry + (ex & 0xFFFFu), ia = acarry + (ex >> 16);
      for (uint32_t r = remw[m]; r; r &= r - 1u, ++ir)
        if (ir < kDiffCap) ps.rem[ir] = 32 * w + __builtin_ctz(r);
      for (uint32_t a = addw[m]; a; a &= a - 1u, ++ia)
        if (ia < kDiffCap) ps.add[ia] = 32 * w + __builtin_ctz(a);
      rcarry += both & 0xFFFFu;
      acarry += both >> 16;
    }
    if (pdiff) atomicAdd(&ps.oldpop, oldpop);
    __syncthreads();
    TopkParams tp{};
    tp.pool = p.pool;
    tp.words = p.words;
    tp.sink = p.sink;
    tp.max_ctx = p.max_ctx;
    const long long cnt_new = (long long)pcnt_old - rcarry + acarry;
    long long count = -1;
    if (pdiff && rcarry <= kDiffCap && acarry <= kDiffCap && ps.oldpop == (uint32_t)pcnt_old &&
        cnt_new <= p.pool.cap)
      count = changes ? pool_apply(tp, ps, pair, b, h, pcnt_old, (int)rcarry, (int)acarry) : pcnt_old;
    if (count < 0) count = pool_rebuild(tp, ps, pair, b, h, n4, mrow);
    // count is the same in every thread; no other thread's store needs to
    // precede the header's (the kernel's end orders them for the readers)
    if (tid == 0) {
      int32_t* phdr = p.pool.header + 4 * (size_t)pair;
      const bool fits = count <= p.pool.cap;
      if (!fits) report_error(p.pool.errors, KVC_ERR_POOL);
      phdr[0] = (int32_t)(fits ? count : p.pool.cap);
      phdr[1] = L;
      phdr[2] = fits ? (int32_t)kPoolMagic : 0;
      phdr[3] = 0;
    }
  }
  if (st && tid == 0) {
    st->magic = kBlockMagic;
    st->len = L;
    st->block = B;
    st->window = p.window;
    st->budget = p.budget;
    st->thr = T;
    st->has_thr = select ? 1 : 0;
    st->gt = (uint32_t)(k - need);
    st->eq = (uint32_t)eqT;
    st->has_cnt = select && by_key ? 1 : 0;
  }
}

template <int B, bool POOL>
__global__ __launch_bounds__(kTopkThreads) void block_topk_kernel(BlockTopkParams p) {
  __shared__ BlockLds sm;
  block_topk_pair<B, POOL>(p, sm, blockIdx.x % p.hkv, blockIdx.x / p.hkv);
}

__global__ __launch_bounds__(kTopkThreads) void topk_kernel(TopkParams p) { topk_group(p, blockIdx.x); }

// workgroups the refresh of a call takes
inline int topk_groups(const TopkParams& p) { return (p.pairs + p.group - 1) / p.group; }

// Scoring and the keep-mask refresh in one launch, for calls that append at
// most 128 positions: the refresh only reads scores of INT4-region positions,
// which lie below L - 128 and so were written by earlier calls. Workgroups
// [0, pairs) refresh one (sequence, kv head) each, or kTopkGroup of them with
// a refresh state (topk_group); the rest score 4 appended rows each (one per
// 256-thread quarter) for one kv head.
template <int D, bool BF16>
__global__ __launch_bounds__(kTopkThreads) void score_topk_kernel(ScoreParams sp, TopkParams tp) {
  __shared__ float xs[kTopkThreads / kScoreThreads][2 * D];
  __shared__ float wsum[kTopkThreads / kScoreThreads][kScoreThreads / 64];
  const int pairs = (tp.pairs + tp.group - 1) / tp.group;  // refresh workgroups
  if ((int)blockIdx.x < pairs) {
    topk_group(tp, blockIdx.x);
    return;
  }
  const int g = blockIdx.x - pairs;
  const int h = g % sp.hkv;
  const int q = threadIdx.x / kScoreThreads;
  const long long f = (long long)(g / sp.hkv) * (kTopkThreads / kScoreThreads) + q;
  ScorerSlice<D> m;
  m.load(sp, h, threadIdx.x % kScoreThreads);
  score_row<D, BF16>(sp, m, h, f, threadIdx.x % kScoreThreads, xs[q], wsum[q]);
}

// The same, with the encoding of the appended rows in the same launch:
// workgroups [pairs, pairs + nq) encode kTopkThreads / 64 (sequence, appended
// token, kv head) items each, one per wave. Nothing the encoding writes is
// read by the refresh or the scorer.
template <int D, bool BF16>
__global__ __launch_bounds__(kTopkThreads) void append_score_topk_kernel(QuantParams qp, ScoreParams sp,
                                                                         TopkParams tp, int nq) {
  __shared__ float xs[kTopkThreads / kScoreThreads][2 * D];
  __shared__ float wsum[kTopkThreads / kScoreThreads][kScoreThreads / 64];
  const int pairs = (tp.pairs + tp.group - 1) / tp.group;  // refresh workgroups
  if ((int)blockIdx.x < pairs) {
    topk_group(tp, blockIdx.x);
    return;
  }
  if ((int)blockIdx.x < pairs + nq) {
    const long long item = (long long)(blockIdx.x - pairs) * (kTopkThreads / 64) + (threadIdx.x >> 6);
    quantize_item<D, BF16>(qp, item, threadIdx.x & 63);
    return;
  }
  const int g = blockIdx.x - pairs - nq;
  const int h = g % sp.hkv;
  const int q = threadIdx.x / kScoreThreads;
  const long long f = (long long)(g / sp.hkv) * (kTopkThreads / kScoreThreads) + q;
  ScorerSlice<D> m;
  m.load(sp, h, threadIdx.x % kScoreThreads);
  score_row<D, BF16>(sp, m, h, f, threadIdx.x % kScoreThreads, xs[q], wsum[q]);
}

}  // namespace

namespace {

ScoreParams score_params(const kvc_cache& c, const float* mlp, const void* k_new, const void* v_new,
                         int n_new_max, const int32_t* n_new) {
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
  // up to 4096 workgroups per head; one row per workgroup at decode
  long long tpg = (total + 4095) / 4096;
  if (tpg < 1) tpg = 1;
  p.tokens_per_group = (int)tpg;
  p.groups_per_head = (int)((total + tpg - 1) / tpg);
  return p;
}

TopkParams topk_params(const kvc_cache& c, int budget_permille, TopkState* state, bool incremental) {
  TopkParams p;
  p.state = state;
  p.incremental = incremental ? 1 : 0;
  p.scores = c.scores;
  p.seq_lens = c.seq_lens;
  p.mask = c.keep_mask;
  p.hkv = c.num_kv_heads;
  p.max_ctx = c.max_ctx;
  p.words = mask_words(c.max_ctx);
  p.budget = budget_permille;
  p.sink = c.n_sink;
  p.recent = c.n_recent;
  p.pool = pool_ref(c);
  p.pairs = c.batch * c.num_kv_heads;
  // A decode step with a state packs pairs (one wave each) into about
  // kTopkResident workgroups; no more per workgroup than that needs, as the
  // pairs of a workgroup that need a full refresh take turns.
  p.group = 1;
  if (incremental && state) {
    const int round = kTopkResident;
    p.group = (p.pairs + round - 1) / round;
    if (p.group > kTopkGroup) p.group = kTopkGroup;
    if (p.group < 1) p.group = 1;
  }
  return p;
}

}  // namespace

hipError_t launch_score(const kvc_cache& c, const float* mlp, const void* k_new, const void* v_new,
                        kvc_dtype src, int n_new_max, const int32_t* n_new, hipStream_t s) {
  const ScoreParams p = score_params(c, mlp, k_new, v_new, n_new_max, n_new);
  const dim3 grid((unsigned)(p.groups_per_head * c.num_kv_heads));
  const bool bf = src == KVC_BF16;
  if (c.head_dim == 128) {
    if (bf) hipLaunchKernelGGL((score_kernel<128, true>), grid, dim3(kScoreThreads), 0, s, p);
    else hipLaunchKernelGGL((score_kernel<128, false>), grid, dim3(kScoreThreads), 0, s, p);
  } else {
    if (bf) hipLaunchKernelGGL((score_kernel<64, true>), grid, dim3(kScoreThreads), 0, s, p);
    else hipLaunchKernelGGL((score_kernel<64, false>), grid, dim3(kScoreThreads), 0, s, p);
  }
  return hipGetLastError();
}

hipError_t launch_topk(const kvc_cache& c, int budget_permille, TopkState* state, bool incremental,
                       hipStream_t s) {
  const TopkParams p = topk_params(c, budget_permille, state, incremental);
  hipLaunchKernelGGL(topk_kernel, dim3((unsigned)topk_groups(p)), dim3(kTopkThreads), 0, s, p);
  return hipGetLastError();
}

template <int D, bool BF16, int B, bool POOL>
__global__ __launch_bounds__(kTopkThreads) void score_block_kernel(ScoreParams sp, BlockTopkParams bp,
                                                                  QuantParams qp, int nq) {
  __shared__ BlockLds sm;
  __shared__ float xs[kTopkThreads / kScoreThreads][2 * D];
  __shared__ float wsum[kTopkThreads / kScoreThreads][kScoreThreads / 64];
  const int pairs = bp.hkv * sp.batch;
  if ((int)blockIdx.x < pairs) {  // the refresh never reads this call's rows: they are protected
    block_topk_pair<B, POOL>(bp, sm, blockIdx.x % bp.hkv, blockIdx.x / bp.hkv);
    return;
  }
  // workgroups [pairs, pairs + nq) encode the appended rows (nq = 0: the
  // caller appended them already), one item per wave
  if ((int)blockIdx.x < pairs + nq) {
    const long long item = (long long)(blockIdx.x - pairs) * (kTopkThreads / 64) + (threadIdx.x >> 6);
    quantize_item<D, BF16>(qp, item, threadIdx.x & 63);
    return;
  }
  const int g = blockIdx.x - pairs - nq;
  const int h = g % sp.hkv;
  const int q = threadIdx.x / kScoreThreads;
  const long long f = (long long)(g / sp.hkv) * (kTopkThreads / kScoreThreads) + q;
  ScorerSlice<D> m;
  m.load(sp, h, threadIdx.x % kScoreThreads);
  score_row<D, BF16>(sp, m, h, f, threadIdx.x % kScoreThreads, xs[q], wsum[q]);
}

static BlockTopkParams block_params(const kvc_cache& c, int budget_permille, int block_tokens,
                                    int window, void* state) {
  BlockTopkParams p;
  p.scores = c.scores;
  p.seq_lens = c.seq_lens;
  p.mask = c.keep_mask;
  p.state = static_cast<unsigned char*>(state);
  p.state_stride = block_state_stride(c);
  p.hkv = c.num_kv_heads;
  p.max_ctx = c.max_ctx;
  p.words = mask_words(c.max_ctx);
  p.budget = budget_permille;
  p.window = window;
  p.sink = c.n_sink;
  p.recent = c.n_recent;
  p.pool = pool_ref(c);
  return p;
}

hipError_t launch_block_topk(const kvc_cache& c, int budget_permille, int block_tokens, int window,
                             void* state, hipStream_t s) {
  const BlockTopkParams p = block_params(c, budget_permille, block_tokens, window, state);
  const dim3 grid(c.batch * c.num_kv_heads), block(kTopkThreads);
  const bool pool = p.pool.cap > 0;
  switch (block_tokens * 2 + (pool ? 1 : 0)) {
    case 32: hipLaunchKernelGGL((block_topk_kernel<16, false>), grid, block, 0, s, p); break;
    case 33: hipLaunchKernelGGL((block_topk_kernel<16, true>), grid, block, 0, s, p); break;
    case 64: hipLaunchKernelGGL((block_topk_kernel<32, false>), grid, block, 0, s, p); break;
    case 65: hipLaunchKernelGGL((block_topk_kernel<32, true>), grid, block, 0, s, p); break;
    case 128: hipLaunchKernelGGL((block_topk_kernel<64, false>), grid, block, 0, s, p); break;
    case 129: hipLaunchKernelGGL((block_topk_kernel<64, true>), grid, block, 0, s, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int D, bool BF16>
static void launch_score_block_d(const dim3& grid, int block_tokens, const ScoreParams& sp,
                                 const BlockTopkParams& bp, const QuantParams& qp, int nq,
                                 hipStream_t s) {
  const dim3 block(kTopkThreads);
  const bool pool = bp.pool.cap > 0;
  if (block_tokens == 16) {
    if (pool) hipLaunchKernelGGL((score_block_kernel<D, BF16, 16, true>), grid, block, 0, s, sp, bp, qp, nq);
    else hipLaunchKernelGGL((score_block_kernel<D, BF16, 16, false>), grid, block, 0, s, sp, bp, qp, nq);
  } else if (block_tokens == 32) {
    if (pool) hipLaunchKernelGGL((score_block_kernel<D, BF16, 32, true>), grid, block, 0, s, sp, bp, qp, nq);
    else hipLaunchKernelGGL((score_block_kernel<D, BF16, 32, false>), grid, block, 0, s, sp, bp, qp, nq);
  } else {
    if (pool) hipLaunchKernelGGL((score_block_kernel<D, BF16, 64, true>), grid, block, 0, s, sp, bp, qp, nq);
    else hipLaunchKernelGGL((score_block_kernel<D, BF16, 64, false>), grid, block, 0, s, sp, bp, qp, nq);
  }
}

hipError_t launch_score_block(const kvc_cache& c, const float* mlp, const void* k_new,
                              const void* v_new, kvc_dtype src, int n_new_max, const int32_t* n_new,
                              int budget_permille, int block_tokens, int window, void* state,
                              bool encode, hipStream_t s) {
  if (block_tokens != 16 && block_tokens != 32 && block_tokens != 64) return hipErrorInvalidValue;
  const ScoreParams sp = score_params(c, mlp, k_new, v_new, n_new_max, n_new);
  const BlockTopkParams bp = block_params(c, budget_permille, block_tokens, window, state);
  const QuantParams qp = quant_params(c, k_new, v_new, n_new_max, n_new);
  const int nq = encode ? (int)((qp.items + kTopkThreads / 64 - 1) / (kTopkThreads / 64)) : 0;
  const long long rows = (long long)c.batch * n_new_max;
  const long long quads = (rows + 3) / 4;
  const dim3 grid((unsigned)((long long)c.batch * c.num_kv_heads + nq + quads * c.num_kv_heads));
  const bool bf = src == KVC_BF16;
  if (c.head_dim == 128) {
    if (bf) launch_score_block_d<128, true>(grid, block_tokens, sp, bp, qp, nq, s);
    else launch_score_block_d<128, false>(grid, block_tokens, sp, bp, qp, nq, s);
  } else {
    if (bf) launch_score_block_d<64, true>(grid, block_tokens, sp, bp, qp, nq, s);
    else launch_score_block_d<64, false>(grid, block_tokens, sp, bp, qp, nq, s);
  }
  return hipGetLastError();
}

hipError_t launch_score_topk(const kvc_cache& c, const float* mlp, const void* k_new,
                             const void* v_new, kvc_dtype src, int n_new_max, const int32_t* n_new,
                             int budget_permille, TopkState* state, hipStream_t s) {
  const ScoreParams sp = score_params(c, mlp, k_new, v_new, n_new_max, n_new);
  const TopkParams tp = topk_params(c, budget_permille, state, true);
  const long long rows = (long long)c.batch * n_new_max;
  const long long quads = (rows + 3) / 4;
  const dim3 grid((unsigned)(topk_groups(tp) + quads * c.num_kv_heads));
  const bool bf = src == KVC_BF16;
  if (c.head_dim == 128) {
    if (bf) hipLaunchKernelGGL((score_topk_kernel<128, true>), grid, dim3(kTopkThreads), 0, s, sp, tp);
    else hipLaunchKernelGGL((score_topk_kernel<128, false>), grid, dim3(kTopkThreads), 0, s, sp, tp);
  } else {
    if (bf) hipLaunchKernelGGL((score_topk_kernel<64, true>), grid, dim3(kTopkThreads), 0, s, sp, tp);
    else hipLaunchKernelGGL((score_topk_kernel<64, false>), grid, dim3(kTopkThreads), 0, s, sp, tp);
  }
  return hipGetLastError();
}

hipError_t launch_append_score_topk(const kvc_cache& c, const float* mlp, const void* k_new,
                                    const void* v_new, kvc_dtype src, int n_new_max,
                                    const int32_t* n_new, int budget_permille, TopkState* state,
                                    hipStream_t s) {
  const QuantParams qp = quant_params(c, k_new, v_new, n_new_max, n_new);
  const ScoreParams sp = score_params(c, mlp, k_new, v_new, n_new_max, n_new);
  const TopkParams tp = topk_params(c, budget_permille, state, true);
  const long long rows = (long long)c.batch * n_new_max;
  const long long quads = mlp ? (rows + 3) / 4 : 0;  // no scoring with the caller's scores
  const int nq = (int)((qp.items + kTopkThreads / 64 - 1) / (kTopkThreads / 64));
  const dim3 grid((unsigned)(topk_groups(tp) + nq + quads * c.num_kv_heads));
  const bool bf = src == KVC_BF16;
  if (c.head_dim == 128) {
    if (bf) hipLaunchKernelGGL((append_score_topk_kernel<128, true>), grid, dim3(kTopkThreads), 0, s, qp, sp, tp, nq);
    else hipLaunchKernelGGL((append_score_topk_kernel<128, false>), grid, dim3(kTopkThreads), 0, s, qp, sp, tp, nq);
  } else {
    if (bf) hipLaunchKernelGGL((append_score_topk_kernel<64, true>), grid, dim3(kTopkThreads), 0, s, qp, sp, tp, nq);
    else hipLaunchKernelGGL((append_score_topk_kernel<64, false>), grid, dim3(kTopkThreads), 0, s, qp, sp, tp, nq);
  }
  return hipGetLastError();
}

}  // namespace kvc
