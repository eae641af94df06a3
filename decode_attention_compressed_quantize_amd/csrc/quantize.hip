// Quantize-on-append launch: one wave per (sequence, appended token, kv
// head), the encoding itself in quant_row.h (KV4-RL review, section 3).
#include "quant_row.h"

// Every product and difference of the encoding rule must round on its own.
#pragma clang fp contract(off)

namespace kvc {
namespace {

template <int D, bool BF16>
__global__ __launch_bounds__(256) void quantize_append_kernel(QuantParams p) {
  quantize_item<D, BF16>(p, (long long)blockIdx.x * 4 + (threadIdx.x >> 6), threadIdx.x & 63);
}

}  // namespace

hipError_t launch_quantize_append(const kvc_cache& c, const void* k_new, const void* v_new,
                                  kvc_dtype src, int n_new_max, const int32_t* n_new,
                                  hipStream_t s) {
  QuantParams p = quant_params(c, k_new, v_new, n_new_max, n_new);
  if (c.pool_capacity > 0) p.pool_header = c.pool_header;
  const dim3 grid((unsigned)((p.items + 3) / 4));
  const dim3 block(256);
  const bool bf = src == KVC_BF16;
  if (c.head_dim == 128) {
    if (bf) hipLaunchKernelGGL((quantize_append_kernel<128, true>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((quantize_append_kernel<128, false>), grid, block, 0, s, p);
  } else {
    if (bf) hipLaunchKernelGGL((quantize_append_kernel<64, true>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((quantize_append_kernel<64, false>), grid, block, 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace kvc
