// Streaming-read probe: the HBM read rate this part reaches with plain wide
// loads, against which the attention kernels' rates are also reported.
//
// Every 32-bit word of the buffer is read once with 16-byte non-temporal loads
// and XOR-folded. Each workgroup streams one contiguous segment, its 256
// threads covering 4 KB per load and kProbeUnroll loads in flight; each
// workgroup XORs its fold into *out, so the result is exact and checkable and
// no load is dead. (Of the patterns tried on MI355X - one segment per wave,
// grid-stride, one segment per workgroup, with and without the non-temporal
// hint - this one reads fastest; the hint is worth about 12%.)
#include "kvc_internal.h"

namespace kvc {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 8;
constexpr size_t kProbeStep = (size_t)kProbeThreads * kProbeUnroll;  // 16-byte items per step

__global__ __launch_bounds__(kProbeThreads) void stream_read_kernel(const u32x4* buf, size_t n16,
                                                                    size_t per, uint32_t* out) {
  // segment of this workgroup: [s0, s1), per a multiple of kProbeStep
  const size_t s0 = (size_t)blockIdx.x * per;
  const size_t s1 = s0 + per < n16 ? s0 + per : n16;
  u32x4 acc = {0u, 0u, 0u, 0u};
  size_t i = s0 + threadIdx.x;
  if (s1 > s0) {
    const size_t full = (s1 - s0) / kProbeStep;  // whole steps, every load in bounds
    for (size_t st = 0; st < full; ++st, i += kProbeStep) {
      u32x4 v[kProbeUnroll];
#pragma unroll
      for (int u = 0; u < kProbeUnroll; ++u) v[u] = __builtin_nontemporal_load(&buf[i + u * kProbeThreads]);
#pragma unroll
      for (int u = 0; u < kProbeUnroll; ++u) acc ^= v[u];
    }
    for (; i < s1; i += kProbeThreads) acc ^= buf[i];
  }
  uint32_t x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x ^= (uint32_t)__shfl_xor((int)x, o);
  __shared__ uint32_t red[kProbeThreads / 64];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
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
  // 2048 workgroups (8 per CU) when the buffer is large; segments of whole steps
  size_t blocks = (n16 + kProbeStep - 1) / kProbeStep;
  if (blocks > 2048) blocks = 2048;
  if (blocks < 1) blocks = 1;
  size_t per = (n16 + blocks - 1) / blocks;
  per = (per + kProbeStep - 1) / kProbeStep * kProbeStep;
  hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)blocks), dim3(kProbeThreads), 0, s,
                     static_cast<const u32x4*>(buf), n16, per, out);
  return hipGetLastError();
}

}  // namespace kvc
