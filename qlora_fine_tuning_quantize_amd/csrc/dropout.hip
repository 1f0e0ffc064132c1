// dropout.hip -- the keep mask of the LoRA dropout as bytes.
//
// The pages train with LoraConfig's lora_dropout on the bypass input; the
// layer draws the mask from a counter (the element index) rather than
// storing it, so forward and backward regenerate the same mask from the
// seed.  This kernel writes that mask out (keep[e] = 1 or 0) for callers
// that want to see it; the layer's own kernels never read it.
#include "kernels.h"

namespace qlora {

// One lane per 16 mask bytes (four Philox draws); the last n % 16 bytes go
// one by one.
__global__ __launch_bounds__(256) void k_dropout_mask(int64_t n, Dropout d,
                                                      uint8_t *__restrict__ keep) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t e0 = 16 * i;
  if (e0 >= n) return;
  if (e0 + 16 <= n) {
    u32x4 o;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t b = dropout_keep4(d, (uint64_t)(e0 + 4 * w));
      o[w] = (b & 1u) | ((b >> 1) & 1u) << 8 | ((b >> 2) & 1u) << 16 | ((b >> 3) & 1u) << 24;
    }
    *reinterpret_cast<u32x4 *>(keep + e0) = o;
  } else {
    for (int64_t e = e0; e < n; e += 4) {
      const uint32_t b = dropout_keep4(d, (uint64_t)e);
      for (int t = 0; t < 4 && e + t < n; ++t) keep[e + t] = (uint8_t)((b >> t) & 1u);
    }
  }
}

int launch_dropout_mask(int64_t M, int64_t K, const Dropout &d, uint8_t *keep,
                        hipStream_t stream) {
  const int64_t n = M * K;
  if (n <= 0) return QL_OK;
  const int64_t lanes = (n + 15) / 16;
  hipLaunchKernelGGL(k_dropout_mask, dim3((unsigned)((lanes + 255) / 256)), dim3(256), 0, stream,
                     n, d, keep);
  QL_HIP_CHECK_LAUNCH();
  return QL_OK;
}

}  // namespace qlora
