// simple.hip -- fp32-accumulating tiled kernels of the layer for any
// activation dtype (the fp32 compute path, and the general fallback).
//
//   forward:  y  = x W^^T + s u B^T      (26. QLoRA and 4bit Quantization, Step 3)
//   backward: dx = dy W^ + g A            (22. QLoRA and 4bit Quantization, Step 1)
//
// W^ is dequantised on the fly (26. ..., Step 4: table[index] * scale) into
// fp32 tiles in LDS; it is never written to global memory.  Tiles are 64x64
// with a contraction step of 64, which for the forward is exactly one
// 64-element chunk of each weight row (one NF4 block, or half of one with
// blocks of 128).
#include "kernels.h"

namespace qlora {

constexpr int kT = 64;

template <typename T>
__device__ __forceinline__ float ldv(const void *p, int64_t i) {
  return load_as_f32(reinterpret_cast<const T *>(p), i);
}

// Forward.  Lane (tm = t / 16, tn = t % 16) owns rows tm*4..+4, cols tn*4..+4.
template <typename AT, typename LT>
__global__ __launch_bounds__(256) void k_simple_fwd(const void *__restrict__ x, int64_t M,
                                                    const uint8_t *__restrict__ packed,
                                                    BlockScales sc, int64_t N, int64_t K,
                                                    const float *__restrict__ u,
                                                    const void *__restrict__ B, int32_t r, float s,
                                                    void *__restrict__ y) {
  __shared__ float xs[kT][kT + 1];
  __shared__ float ws[kT][kT + 1];
  __shared__ float cb[16];
  const int t = threadIdx.x;
  if (t < 16) cb[t] = c_nf4[t];
  const int64_t m0 = (int64_t)blockIdx.y * kT, n0 = (int64_t)blockIdx.x * kT;
  const int tm = t / 16, tn = t % 16;
  float acc[4][4] = {};
  const int64_t kb_per_row = K / 64;
  for (int64_t k0 = 0; k0 < K; k0 += kT) {
    for (int e = t; e < kT * kT; e += 256) {
      const int rr = e / kT, cc = e % kT;
      const int64_t m = m0 + rr;
      xs[rr][cc] = (m < M) ? ldv<AT>(x, m * K + k0 + cc) : 0.0f;
    }
    __syncthreads();  // also publishes cb on the first pass
    {
      // lane t dequantises 16 consecutive weights of row t / 4
      const int rr = t / 4, part = t % 4;
      const int64_t n = n0 + rr;
      if (n < N) {
        const float a = sc(n * kb_per_row + k0 / 64);
        const uint8_t *src = packed + ((n * K + k0) >> 1) + part * 8;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const uint8_t byte = src[i];
          ws[rr][part * 16 + 2 * i] = cb[byte >> 4] * a;
          ws[rr][part * 16 + 2 * i + 1] = cb[byte & 15] * a;
        }
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) ws[rr][part * 16 + i] = 0.0f;
      }
    }
    __syncthreads();
    for (int kk = 0; kk < kT; ++kk) {
      float av[4], bv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) av[i] = xs[tm * 4 + i][kk];
#pragma unroll
      for (int j = 0; j < 4; ++j) bv[j] = ws[tn * 4 + j][kk];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_fmaf(av[i], bv[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t m = m0 + tm * 4 + i;
    if (m >= M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t n = n0 + tn * 4 + j;
      if (n >= N) continue;
      float l = 0.0f;
      for (int jj = 0; jj < r; ++jj) l = __builtin_fmaf(u[m * r + jj], ldv<LT>(B, n * r + jj), l);
      store_from_f32(reinterpret_cast<AT *>(y), m * N + n, __builtin_fmaf(s, l, acc[i][j]));
    }
  }
}

// Input gradient.  Contraction over n in steps of 64; the weight tile holds
// rows n0..n0+64 of W^ restricted to columns k0..k0+64 (one 64-element
// chunk of each row, inside one NF4 block).
// DROP: LoRA dropout on the bypass input; the bypass term of output (m, k)
// is multiplied by keep(m, k) / (1 - p) (dscale) before the base product is
// added to it.
template <typename AT, typename LT, bool DROP>
__global__ __launch_bounds__(256) void k_simple_dx(const void *__restrict__ dy, int64_t M,
                                                   const uint8_t *__restrict__ packed,
                                                   BlockScales sc, int64_t N, int64_t K,
                                                   const float *__restrict__ g,
                                                   const void *__restrict__ A, int32_t r,
                                                   void *__restrict__ dx, Dropout dr,
                                                   float dscale) {
  __shared__ float ds[kT][kT + 1];  // [m][n]
  __shared__ float ws[kT][kT + 1];  // [n][k]
  __shared__ float cb[16];
  const int t = threadIdx.x;
  if (t < 16) cb[t] = c_nf4[t];
  const int64_t m0 = (int64_t)blockIdx.y * kT, k0 = (int64_t)blockIdx.x * kT;
  const int tm = t / 16, tk = t % 16;
  float acc[4][4] = {};
  const int64_t kb_per_row = K / 64;
  for (int64_t n0 = 0; n0 < N; n0 += kT) {
    for (int e = t; e < kT * kT; e += 256) {
      const int rr = e / kT, cc = e % kT;
      const int64_t m = m0 + rr, n = n0 + cc;
      ds[rr][cc] = (m < M && n < N) ? ldv<AT>(dy, m * N + n) : 0.0f;
    }
    __syncthreads();
    {
      const int rr = t / 4, part = t % 4;
      const int64_t n = n0 + rr;
      if (n < N) {
        const float a = sc(n * kb_per_row + k0 / 64);
        const uint8_t *src = packed + ((n * K + k0) >> 1) + part * 8;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const uint8_t byte = src[i];
          ws[rr][part * 16 + 2 * i] = cb[byte >> 4] * a;
          ws[rr][part * 16 + 2 * i + 1] = cb[byte & 15] * a;
        }
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) ws[rr][part * 16 + i] = 0.0f;
      }
    }
    __syncthreads();
    for (int nn = 0; nn < kT; ++nn) {
      float av[4], bv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) av[i] = ds[tm * 4 + i][nn];
#pragma unroll
      for (int j = 0; j < 4; ++j) bv[j] = ws[nn][tk * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_fmaf(av[i], bv[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t m = m0 + tm * 4 + i;
    if (m >= M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t k = k0 + tk * 4 + j;
      float l = 0.0f;
      for (int jj = 0; jj < r; ++jj) l = __builtin_fmaf(g[m * r + jj], ldv<LT>(A, jj * K + k), l);
      if constexpr (DROP) l = dropout_keep1(dr, (uint64_t)(m * K + k)) ? dscale * l : 0.0f;
      store_from_f32(reinterpret_cast<AT *>(dx), m * K + k, acc[i][j] + l);
    }
  }
}

int launch_simple_fwd(const void *x, int act_dtype, int64_t M, const uint8_t *packed,
                      BlockScales sc, int64_t N, int64_t K, const float *u, const void *B,
                      int lora_dtype, int32_t r, float s, void *y, hipStream_t stream) {
  const dim3 grid((unsigned)((N + kT - 1) / kT), (unsigned)((M + kT - 1) / kT));
  with_type(act_dtype, [&](auto *at) {
    with_type(lora_dtype, [&](auto *lt) {
      hipLaunchKernelGGL((k_simple_fwd<elem_of<decltype(at)>, elem_of<decltype(lt)>>), grid,
                         dim3(256), 0, stream, x, M, packed, sc, N, K, u, B, r, s, y);
    });
  });
  QL_HIP_CHECK_LAUNCH();
  return QL_OK;
}

int launch_simple_dx(const void *dy, int act_dtype, int64_t M, const uint8_t *packed,
                     BlockScales sc, int64_t N, int64_t K, const float *g, const void *A,
                     int lora_dtype, int32_t r, void *dx, hipStream_t stream,
                     const Dropout *drop, float dscale) {
  const dim3 grid((unsigned)(K / kT), (unsigned)((M + kT - 1) / kT));
  const Dropout dr = drop ? *drop : Dropout{0u, 0u, 0u};
  with_type(act_dtype, [&](auto *at) {
    with_type(lora_dtype, [&](auto *lt) {
      using AT = elem_of<decltype(at)>;
      using LT = elem_of<decltype(lt)>;
      if (drop)
        hipLaunchKernelGGL((k_simple_dx<AT, LT, true>), grid, dim3(256), 0, stream, dy, M, packed,
                           sc, N, K, g, A, r, dx, dr, dscale);
      else
        hipLaunchKernelGGL((k_simple_dx<AT, LT, false>), grid, dim3(256), 0, stream, dy, M,
                           packed, sc, N, K, g, A, r, dx, dr, 1.0f);
    });
  });
  QL_HIP_CHECK_LAUNCH();
  return QL_OK;
}

}  // namespace qlora
