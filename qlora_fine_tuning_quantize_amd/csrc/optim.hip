// optim.hip -- one AdamW step over the LoRA factors, in place.
//
// The pages train the LoRA factors with AdamW holding fp32 moments (gufacode
// fine-tuning chapter 4, "显存计算实战" and "分页优化器": 8 bytes per
// trainable parameter; Gemma lesson 9, sec. 9.4: two states per parameter).
// The update is the published AdamW definition (decoupled weight decay,
// bias-corrected moments), each operation one fp32 rounding, none fused:
//   p = p * decay;  m = b1 m + (1 - b1) g;  v = b2 v + (1 - b2) (g g)
//   p = p - step_size * (m / (sqrt(v) / bc2_sqrt + eps))
// The scalars (decay = 1 - lr wd, step_size = lr / (1 - b1^t), bc2_sqrt =
// sqrt(1 - b2^t)) are computed once on the host.  HBM-bound: per parameter
// 16 bytes read (p, g, m, v) and 12 written (p, m, v), +2 for the optional
// bf16 copy of p that the layer reads.
#include <cmath>

#include "kernels.h"

namespace qlora {

#pragma clang fp contract(off)

struct AdamScalars {
  float decay, b1, omb1, b2, omb2, eps, step_size, bc2_sqrt;
};

__device__ __forceinline__ void adam_one(float &p, float g, float &m, float &v,
                                         const AdamScalars &a) {
  float pi = p * a.decay;
  const float mi = a.b1 * m + a.omb1 * g;
  const float gg = g * g;
  const float vi = a.b2 * v + a.omb2 * gg;
  const float denom = __builtin_sqrtf(vi) / a.bc2_sqrt + a.eps;
  const float upd = mi / denom;
  pi = pi - a.step_size * upd;
  p = pi;
  m = mi;
  v = vi;
}

// 4 parameters per lane with 16-byte accesses; the last n % 4 go one by one.
__global__ __launch_bounds__(256) void k_adamw(float *__restrict__ p, const float *__restrict__ g,
                                               float *__restrict__ m, float *__restrict__ v,
                                               uint16_t *__restrict__ p_bf16, int64_t n,
                                               AdamScalars a) {
  const int64_t n4 = n >> 2;
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += stride) {
    f32x4 pv = reinterpret_cast<f32x4 *>(p)[i];
    const f32x4 gv = reinterpret_cast<const f32x4 *>(g)[i];
    f32x4 mv = reinterpret_cast<f32x4 *>(m)[i];
    f32x4 vv = reinterpret_cast<f32x4 *>(v)[i];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float pe = pv[e], me = mv[e], ve = vv[e];
      adam_one(pe, gv[e], me, ve, a);
      pv[e] = pe;
      mv[e] = me;
      vv[e] = ve;
    }
    reinterpret_cast<f32x4 *>(p)[i] = pv;
    reinterpret_cast<f32x4 *>(m)[i] = mv;
    reinterpret_cast<f32x4 *>(v)[i] = vv;
    if (p_bf16)
      reinterpret_cast<u32x2 *>(p_bf16)[i] = u32x2{pack_bf16x2(pv[0], pv[1]), pack_bf16x2(pv[2], pv[3])};
  }
  if (blockIdx.x == 0 && threadIdx.x < (n & 3)) {
    const int64_t i = 4 * n4 + threadIdx.x;
    float pe = p[i], me = m[i], ve = v[i];
    adam_one(pe, g[i], me, ve, a);
    p[i] = pe;
    m[i] = me;
    v[i] = ve;
    if (p_bf16) p_bf16[i] = f32_to_bf16_bits(pe);
  }
}

int launch_adamw(float *p, const float *g, float *m, float *v, uint16_t *p_bf16, int64_t n,
                 double lr, double beta1, double beta2, double eps, double weight_decay,
                 int64_t step, hipStream_t stream) {
  if (n <= 0) return QL_OK;
  AdamScalars a;
  a.decay = (float)(1.0 - lr * weight_decay);
  a.b1 = (float)beta1;
  a.omb1 = (float)(1.0 - beta1);
  a.b2 = (float)beta2;
  a.omb2 = (float)(1.0 - beta2);
  a.eps = (float)eps;
  a.step_size = (float)(lr / (1.0 - std::pow(beta1, (double)step)));
  a.bc2_sqrt = (float)std::sqrt(1.0 - std::pow(beta2, (double)step));
  const int64_t n4 = n >> 2;
  int64_t blocks = (n4 + 255) / 256;
  if (blocks < 1) blocks = 1;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(k_adamw, dim3((unsigned)blocks), dim3(256), 0, stream, p, g, m, v, p_bf16, n, a);
  QL_HIP_CHECK_LAUNCH();
  return QL_OK;
}

}  // namespace qlora
