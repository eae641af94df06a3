// Streaming-read probe: the HBM read rate this part reaches on a plain
// streaming pattern, against which the attention kernels' rates are also
// reported.
//
// Every 32-bit word of the buffer is read once with 16-byte non-temporal
// direct-to-LDS loads and XOR-folded. Each workgroup streams one contiguous
// segment; each workgroup XORs its fold into *out, so the result is exact and
// checkable and no load is dead. On MI355X the rate falls as more bytes are in
// flight: about 8 MB chip-wide (kProbeBlocks workgroups of four waves with two
// 1 KB pieces each) read fastest, 7.0-7.1 TB/s; 16, 32 and 64 MB read 7%, 12%
// and 14% slower (a version loading into registers with 64 MB in flight read
// 6.1 TB/s).
#include "kvc_internal.h"

namespace kvc {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kProbeThreads = 256;
constexpr size_t kProbeStep = (size_t)kProbeThreads * 8;  // 16-byte items per segment step (32 KB)
constexpr int kProbeBlocks = 1024;                         // four per CU
constexpr int kDmaBuf = 2;                                 // 1 KB buffers per wave

// Each wave streams 1 KB pieces (64 lanes x 16 bytes, non-temporal) of its
// workgroup's segment through a ring of kDmaBuf LDS buffers filled by
// direct-to-LDS loads (the attention kernels' pattern) and XORs each piece out
// of LDS once it has landed; the wait before a piece counts exactly the pieces
// issued after it.

template <int N>
__device__ inline u32x4 lds_read_after_n(uint32_t lds) {
  u32x4 v;
  asm volatile("s_waitcnt vmcnt(%1)\n\tds_read_b128 %0, %2\n\ts_waitcnt lgkmcnt(0)"
               : "=&v"(v)
               : "n"(N), "v"(lds)
               : "memory");
  return v;
}

template <int N>
__device__ inline u32x4 lds_read_after(int after, uint32_t lds) {
  if constexpr (N == 0) {
    return lds_read_after_n<0>(lds);
  } else {
    if (after >= N) return lds_read_after_n<N>(lds);
    return lds_read_after<N - 1>(after, lds);
  }
}

__global__ __launch_bounds__(kProbeThreads) void stream_read_dma_kernel(const u32x4* buf, size_t n16,
                                                                        size_t per, uint32_t* out) {
  __shared__ u32x4 ring[kProbeThreads / 64][kDmaBuf][64];
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const size_t s0 = (size_t)blockIdx.x * per;
  const size_t s1 = s0 + per < n16 ? s0 + per : n16;
  const size_t n = s1 > s0 ? s1 - s0 : 0;
  const size_t pieces = n / 64;  // whole pieces; wave w takes pieces w, w + 4, ...
  const size_t nw = pieces > (size_t)wave ? (pieces - wave + 3) / 4 : 0;
  const uint32_t lds0 = (uint32_t)(uintptr_t)&ring[wave][0][0];
  auto issue = [&](size_t j, int k) {
    __builtin_amdgcn_global_load_lds(buf + s0 + (wave + 4 * j) * 64 + lane,
                                     (__attribute__((address_space(3))) void*)&ring[wave][k][0], 16, 0, 2);
  };
  u32x4 acc = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int k = 0; k < kDmaBuf; ++k)
    if ((size_t)k < nw) issue(k, k);
  for (size_t j = 0; j < nw; ++j) {
    const int k = (int)(j % kDmaBuf);
    const size_t left = nw - 1 - j;  // pieces of this wave still to come
    acc ^= lds_read_after<kDmaBuf - 1>(left < (size_t)(kDmaBuf - 1) ? (int)left : kDmaBuf - 1,
                                       lds0 + (uint32_t)(k * 64 + lane) * 16u);
    if (j + kDmaBuf < nw) issue(j + kDmaBuf, k);
  }
  // the items past the whole pieces, with plain loads
  for (size_t i = s0 + pieces * 64 + threadIdx.x; i < s1; i += kProbeThreads) acc ^= buf[i];
  uint32_t x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x ^= (uint32_t)__shfl_xor((int)x, o);
  __shared__ uint32_t red[kProbeThreads / 64];
  if (lane == 0) red[wave] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t y = 0;
#pragma unroll
    for (int w = 0; w < kProbeThreads / 64; ++w) y ^= red[w];
    atomicXor(out, y);
  }
}

}  // namespace

hipError_t launch_stream_read(const void* buf, size_t bytes, uint32_t* out, hipStream_t s) {
  const size_t n16 = bytes / 16;
  // kProbeBlocks workgroups when the buffer is large; segments of whole steps
  size_t blocks = (n16 + kProbeStep - 1) / kProbeStep;
  if (blocks > (size_t)kProbeBlocks) blocks = kProbeBlocks;
  if (blocks < 1) blocks = 1;
  size_t per = (n16 + blocks - 1) / blocks;
  per = (per + kProbeStep - 1) / kProbeStep * kProbeStep;
  hipLaunchKernelGGL(stream_read_dma_kernel, dim3((unsigned)blocks), dim3(kProbeThreads), 0, s,
                     static_cast<const u32x4*>(buf), n16, per, out);
  return hipGetLastError();
}

}  // namespace kvc
