// upart.h -- u = x A^T in slices, the rank-r down projection of the
// QLoRA bypass (26. QLoRA and 4bit Quantization, Step 3), for launches that
// compute u in some of their own workgroups and leave the sum of the slices
// to a later launch.
#pragma once
#include "common.h"

namespace qlora {

constexpr int kUChunk = 128;      // contraction columns per chunk
constexpr int kUMaxSlices = 16;   // contraction slices of u at most

// 8 16-bit values of a LoRA-A row as a matrix-core operand in format AT
template <typename AT, typename LT>
__device__ __forceinline__ u32x4 lora_op8(const LT *p) {
  if constexpr (sizeof(LT) == 2) {
    return *reinterpret_cast<const u32x4 *>(p);
  } else {
    const float4 a = reinterpret_cast<const float4 *>(p)[0];
    const float4 b = reinterpret_cast<const float4 *>(p)[1];
    return u32x4{Half<AT>::pack2(a.x, a.y), Half<AT>::pack2(a.z, a.w), Half<AT>::pack2(b.x, b.y),
                 Half<AT>::pack2(b.z, b.w)};
  }
}

// u = x A^T for token rows [16 tg, 16 tg + 16), rank tile jt (16 ranks),
// over the contraction chunks [su uc, su uc + uc), summed over the
// workgroup's 4 waves: upart[su][m][16 jt + j].  256 threads; red: 4 x 16 x
// 16 floats of LDS.  K % 32 == 0.  Rows past M and ranks past r repeat the
// last valid one and are not stored.  With LoRA dropout (dr.thr != 0) the
// dropped elements of x are zeroed as loaded; the 1 / (1 - p) scale is left
// to the launch that sums the slices.
template <typename AT, typename LT>
__device__ __forceinline__ void u_slice_tile(const uint16_t *__restrict__ x, int M, int64_t K,
                                             const LT *__restrict__ A, int32_t r,
                                             float *__restrict__ upart, int uc, int su, int jt,
                                             int tg, float *red, Dropout dr) {
  constexpr int kWaves = 4;
  const int t = threadIdx.x;
  const int wave = t >> 6, lane = t & 63;
  const int nl = lane & 15, q = lane >> 4;
  const int m = 16 * tg + nl < M ? 16 * tg + nl : M - 1;
  const int64_t col0 = (int64_t)su * uc * kUChunk;
  const int64_t col1 = col0 + (int64_t)uc * kUChunk < K ? col0 + (int64_t)uc * kUChunk : K;
  const int nsteps = (int)((col1 - col0) / 32);
  const int j = 16 * jt + nl < r ? 16 * jt + nl : r - 1;
  const uint16_t *xp = x + (int64_t)m * K + col0 + 8 * q;
  const LT *ap = A + (int64_t)j * K + col0 + 8 * q;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  // steps wave, wave + 4, ...: four at a time, all their loads issued
  // before the first op (clamped to a valid step; extra ones not used)
  for (int s0 = wave; s0 < nsteps; s0 += 4 * kWaves) {
    u32x4 xo[4], ao[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int st = s0 + kWaves * i < nsteps ? s0 + kWaves * i : s0;
      xo[i] = *reinterpret_cast<const u32x4 *>(xp + 32 * st);
      ao[i] = lora_op8<AT>(ap + 32 * st);
    }
    if (dr.thr != 0u) {  // uniform
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int st = s0 + kWaves * i < nsteps ? s0 + kWaves * i : s0;
        xo[i] = dropout_mask8(dr, (uint64_t)m * K + col0 + 8 * q + 32 * st, xo[i]);
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (s0 + kWaves * i < nsteps) acc = Half<AT>::mfma16(xo[i], ao[i], acc);
  }
  // acc[v] = partial u[16 tg + 4q + v][16 jt + nl]
#pragma unroll
  for (int v = 0; v < 4; ++v) red[(wave * 16 + 4 * q + v) * 16 + nl] = acc[v];
  __syncthreads();
  const int mo = t >> 4, jj = t & 15;
  if (16 * tg + mo < M) {
    float sum = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) sum += red[(w * 16 + mo) * 16 + jj];
    if (16 * jt + jj < r) upart[((int64_t)su * M + 16 * tg + mo) * r + 16 * jt + jj] = sum;
  }
}

// Slices of u over a contraction of NC = ceil(K / 128) chunks: one slice per
// 4 chunks, at most kUMaxSlices; uc chunks each.
struct USlices {
  int U, uc;
};
inline USlices u_slices(int64_t K) {
  const int64_t NC = (K + kUChunk - 1) / kUChunk;
  int64_t U = (NC + 3) / 4;
  if (U > kUMaxSlices) U = kUMaxSlices;
  USlices p;
  p.uc = (int)((NC + U - 1) / U);
  p.U = (int)((NC + p.uc - 1) / p.uc);
  return p;
}

}  // namespace qlora
