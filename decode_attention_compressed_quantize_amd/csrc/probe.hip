// Streaming-read probe: the HBM read rate this part reaches with plain wide
// loads, against which the attention kernels' rates are also reported.
//
// Every 32-bit word of the buffer is read once with 16-byte loads (each wave
// streams its own contiguous segment, 8 KB loading while the previous 8 KB
// folds) and XOR-folded; each workgroup XORs its
// fold into *out, so the result is exact and checkable and no load is dead.
#include "kvc_internal.h"

namespace kvc {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 8;

__global__ __launch_bounds__(kProbeThreads) void stream_read_kernel(const u32x4* buf, size_t n16,
                                                                    uint32_t* out) {
  // the buffer is cut into one contiguous segment per wave (whole 1 KB pieces);
  // each wave streams its own segment, kProbeUnroll pieces per step
  const int lane = threadIdx.x & 63;
  const size_t waves = (size_t)gridDim.x * (kProbeThreads / 64);
  const size_t wave = (size_t)blockIdx.x * (kProbeThreads / 64) + (threadIdx.x >> 6);
  const size_t pieces = (n16 + 63) / 64;
  const size_t per = (pieces + waves - 1) / waves;
  const size_t p0 = wave * per, p1 = p0 + per < pieces ? p0 + per : pieces;
  u32x4 acc = {0u, 0u, 0u, 0u};
  // two register sets: the next kProbeUnroll pieces load while this set folds
  auto load = [&](size_t q, u32x4 (&v)[kProbeUnroll]) {
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) v[u] = buf[(q + u) * 64 + lane];
  };
  auto fold = [&](const u32x4 (&v)[kProbeUnroll]) {
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) acc ^= v[u];
  };
  const size_t full = p1 > p0 ? (p1 - p0) / kProbeUnroll : 0;  // whole steps, all in bounds
  if (full > 0 && (p0 + full * kProbeUnroll) * 64 <= n16) {
    // the loads are unconditional (past the last step they repeat it, unused)
    // so that each fold waits only for its own set
    auto step = [&](size_t st) { return p0 + (st < full ? st : full - 1) * kProbeUnroll; };
    u32x4 va[kProbeUnroll], vb[kProbeUnroll];
    load(step(0), va);
    for (size_t st = 1;; st += 2) {
      load(step(st), vb);
      fold(va);
      if (st >= full) break;
      load(step(st + 1), va);
      fold(vb);
      if (st + 1 >= full) break;
    }
  }
  size_t q = full > 0 && (p0 + full * kProbeUnroll) * 64 <= n16 ? p0 + full * kProbeUnroll : p0;
  for (; q < p1; ++q) {
    const size_t i = q * 64 + lane;
    if (i < n16) acc ^= buf[i];
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
  size_t blocks = (n16 + kProbeThreads * kProbeUnroll - 1) / (kProbeThreads * kProbeUnroll);
  if (blocks > 2048) blocks = 2048;  // one resident round at 8 waves per SIMD
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)blocks), dim3(kProbeThreads), 0, s,
                     static_cast<const u32x4*>(buf), n16, out);
  return hipGetLastError();
}

}  // namespace kvc
