// The kept-record pool: per (sequence, kv head) a compact copy of the INT4
// records (codes and fp16 group meta) of the kept INT4-region positions.
//
// Source: KV4-RL review, section 3 - attention reads the INT4 store for the
// body of the context; Shadow Mask Distillation page, Figure 1 caption - a
// binary mask of retained indices decides which positions are attended. The
// pool holds exactly the records the mask keeps, so attention reads 40*D
// bytes per kept token and nothing else, in long contiguous runs.
//
// Layout. Records live in tiles of 32 (40*D bytes), in the order of bytes the
// attention kernel's lanes consume, so that every read of a tile is a run of
// 16-byte (or 8-byte) pieces, one per lane, in lane order. For token t of a
// tile, h(t) = t / 16, s(t) = (t mod 16) / 4 and j(t) = t mod 4: the MFMA rows
// of lane row slot s hold tokens 4s + j and 16 + 4s + j, the lane's eight
// tokens, i = 4h + j:
//   KC [16D bytes]  K codes: piece (h, s, t mod 16) holds K-code bytes
//                   [s*D/8, (s+1)*D/8) of token t (so lane 16s + n reads the
//                   pieces of tokens n and 16 + n at offsets lane and 64 + lane)
//   KM [4D]         K meta: dword ((h*4 + s)*NG + g)*4 + j = (scale | min << 16)
//                   of K group g of token t (NG = D/32 groups)
//   VC [16D]        V codes: dword ((h*4 + s)*VD + d)*4 + j = V-code dword d of
//                   token t (VD = D/8 dwords)
//   VM [4D]         V meta, as KM
// A record is copied into the pool as 16-byte source chunks: its D/2 K-code
// bytes, D/2 V-code bytes and D/4 meta bytes (K groups, then V groups).
//
// Maps (pool_slot, per pair max_ctx + cap entries): entry pos holds the slot of
// a kept INT4-region position, entry max_ctx + slot the position in a slot.
#pragma once

#include "kvc_internal.h"

namespace kvc {

constexpr int kPoolTile = 32;
constexpr uint32_t kPoolMagic = 0x4B565031u;

__host__ __device__ inline int pool_tile_bytes(int D) { return 40 * D; }
__host__ __device__ inline size_t pool_pair_bytes(int D, int cap) {
  return (size_t)(cap / kPoolTile) * pool_tile_bytes(D);
}

// Offsets within a tile (D = 64 or 128).
__device__ inline int pool_row(int t) { return ((t >> 4) << 2) + ((t & 15) >> 2); }  // h*4 + s
__device__ inline int pool_kcode(int D, int t, int s) {
  return (((t >> 4) * 64) + s * 16 + (t & 15)) * (D / 8);
}
__device__ inline int pool_kmeta(int D, int t, int g) {
  return 16 * D + ((pool_row(t) * (D / 32) + g) * 4 + (t & 3)) * 4;
}
__device__ inline int pool_vcode(int D, int t, int d) {
  return 20 * D + ((pool_row(t) * (D / 8) + d) * 4 + (t & 3)) * 4;
}
__device__ inline int pool_vmeta(int D, int t, int g) {
  return 36 * D + ((pool_row(t) * (D / 32) + g) * 4 + (t & 3)) * 4;
}

// What the pool writers need of a cache.
struct PoolRef {
  uint8_t* pool;
  int32_t* slot;
  int32_t* header;
  int cap;  // records per (sequence, kv head); 0: no pool
  const uint8_t* codes;
  const uint16_t* meta;
  const uint8_t* codes_h;
  const uint16_t* meta_h;
  const int32_t* block_table;
  uint32_t* errors;
  int max_pages;
  int num_pages;
  int host_pages;
  int hkv;
  int D;
  int max_ctx;
};

inline PoolRef pool_ref(const kvc_cache& c) {
  PoolRef r;
  r.pool = c.pool;
  r.slot = c.pool_slot;
  r.header = c.pool_header;
  r.cap = c.pool_capacity;
  r.codes = c.int4_codes;
  r.meta = c.int4_meta;
  r.codes_h = c.int4_codes_host;
  r.meta_h = c.int4_meta_host;
  r.block_table = c.block_table;
  r.errors = c.errors;
  r.max_pages = c.max_pages_per_seq;
  r.num_pages = c.num_phys_pages;
  r.host_pages = c.num_host_pages;
  r.hkv = c.num_kv_heads;
  r.D = c.head_dim;
  r.max_ctx = c.max_ctx;
  return r;
}

__device__ inline void report_error(uint32_t* errors, uint32_t bit) {
  if (errors) __hip_atomic_fetch_or(errors, bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The page holding position pos of sequence b, or -1 (with KVC_ERR_PAGE
// reported) when the table entry is outside both page pools.
__device__ inline int pool_page(const PoolRef& r, int b, int pos) {
  const int page = r.block_table[(size_t)b * r.max_pages + (pos >> 4)];
  if (page < 0 || page >= r.num_pages + r.host_pages) {
    report_error(r.errors, KVC_ERR_PAGE);
    return -1;
  }
  return page;
}

// Source chunk c (16 bytes) of the INT4 record of position pos on `page`.
__device__ inline const uint8_t* pool_src_chunk(const PoolRef& r, int page, int kvh, int pos, int c) {
  const bool host = page >= r.num_pages;
  const int pg = host ? page - r.num_pages : page;
  const size_t rec = ((size_t)pg * r.hkv + kvh) * kPage + (pos & 15);
  const int ncode = r.D / 16;
  if (c < ncode) return (host ? r.codes_h : r.codes) + rec * r.D + 16 * c;
  const uint8_t* m = reinterpret_cast<const uint8_t*>(host ? r.meta_h : r.meta);
  return m + rec * (r.D / 4) + 16 * (c - ncode);
}

// Stores source chunk c (loaded into x) of a record into token t of `tile`.
__device__ inline void pool_put_chunk(uint8_t* tile, int D, int t, int c, uint4 x) {
  const int ncode = D / 16;
  if (c < ncode / 2) {  // K codes: one (D = 128) or two (D = 64) lane pieces
    if (D == 128) {
      *reinterpret_cast<uint4*>(tile + pool_kcode(D, t, c)) = x;
    } else {
      *reinterpret_cast<uint2*>(tile + pool_kcode(D, t, 2 * c)) = make_uint2(x.x, x.y);
      *reinterpret_cast<uint2*>(tile + pool_kcode(D, t, 2 * c + 1)) = make_uint2(x.z, x.w);
    }
  } else if (c < ncode) {  // V codes: dwords 4c'..4c'+3
    const int d0 = 4 * (c - ncode / 2);
    *reinterpret_cast<uint32_t*>(tile + pool_vcode(D, t, d0)) = x.x;
    *reinterpret_cast<uint32_t*>(tile + pool_vcode(D, t, d0 + 1)) = x.y;
    *reinterpret_cast<uint32_t*>(tile + pool_vcode(D, t, d0 + 2)) = x.z;
    *reinterpret_cast<uint32_t*>(tile + pool_vcode(D, t, d0 + 3)) = x.w;
  } else {  // meta dwords 4m..4m+3: K groups, then V groups
    const int NG = D / 32;
    const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int md = 4 * (c - ncode) + j;
      const int off = md < NG ? pool_kmeta(D, t, md) : pool_vmeta(D, t, md - NG);
      *reinterpret_cast<uint32_t*>(tile + off) = w[j];
    }
  }
}

__device__ inline int pool_chunks(int D) { return D / 16 + D / 64; }

__device__ inline uint8_t* pool_tile(const PoolRef& r, int pair, int slot) {
  return r.pool + (size_t)pair * pool_pair_bytes(r.D, r.cap) + (size_t)(slot / kPoolTile) * pool_tile_bytes(r.D);
}

// The two maps of a pair.
__device__ inline int32_t* pool_slot_of(const PoolRef& r, int pair) {
  return r.slot + (size_t)pair * ((size_t)r.max_ctx + r.cap);
}
__device__ inline int32_t* pool_pos_of(const PoolRef& r, int pair) {
  return pool_slot_of(r, pair) + r.max_ctx;
}

// Offset within a tile of piece c (0 <= c < 4 + VD + 2 NG) of token t: the
// four K-code pieces (D/8 bytes each), then the V-code dwords, the K meta
// dwords and the V meta dwords (4 bytes each).
__device__ inline int pool_piece(int D, int t, int c) {
  const int VD = D / 8, NG = D / 32;
  if (c < 4) return pool_kcode(D, t, c);
  c -= 4;
  if (c < VD) return pool_vcode(D, t, c);
  c -= VD;
  if (c < NG) return pool_kmeta(D, t, c);
  return pool_vmeta(D, t, c - NG);
}

// Moves the record in slot `from` to slot `to` of the same pair, one thread.
__device__ inline void pool_move_thread(const PoolRef& r, int pair, int from, int to) {
  const uint8_t* src = pool_tile(r, pair, from);
  uint8_t* dst = pool_tile(r, pair, to);
  const int tf = from % kPoolTile, tt = to % kPoolTile;
  const int D = r.D, n = 4 + D / 8 + D / 16;
  for (int c = 0; c < 4; ++c) {  // K-code pieces of D/8 bytes
    if (D == 128)
      *reinterpret_cast<uint4*>(dst + pool_piece(D, tt, c)) =
          *reinterpret_cast<const uint4*>(src + pool_piece(D, tf, c));
    else
      *reinterpret_cast<uint2*>(dst + pool_piece(D, tt, c)) =
          *reinterpret_cast<const uint2*>(src + pool_piece(D, tf, c));
  }
  for (int c = 4; c < n; ++c)  // dword pieces
    *reinterpret_cast<uint32_t*>(dst + pool_piece(D, tt, c)) =
        *reinterpret_cast<const uint32_t*>(src + pool_piece(D, tf, c));
}

// Copies the record of position pos (on `page`) into `slot`, one thread.
__device__ inline void pool_copy_thread(const PoolRef& r, int pair, int kvh, int page, int pos, int slot) {
  uint8_t* tile = pool_tile(r, pair, slot);
  const int t = slot % kPoolTile;
  const int n = pool_chunks(r.D);
  for (int c = 0; c < n; ++c)
    pool_put_chunk(tile, r.D, t, c, *reinterpret_cast<const uint4*>(pool_src_chunk(r, page, kvh, pos, c)));
}

// The same with one wave: lane c copies chunk c.
__device__ inline void pool_copy_wave(const PoolRef& r, int pair, int kvh, int page, int pos, int slot,
                                      int lane) {
  if (lane < pool_chunks(r.D)) {
    const uint4 x = *reinterpret_cast<const uint4*>(pool_src_chunk(r, page, kvh, pos, lane));
    pool_put_chunk(pool_tile(r, pair, slot), r.D, slot % kPoolTile, lane, x);
  }
}

}  // namespace kvc
