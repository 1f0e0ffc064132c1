// tiny.hip -- the fp32 layer for sizes where the tiled fp32 path is all
// launch and round-trip latency (the pages' small fp32 configuration: W
// 256x256, 4 tokens, r = 8, 26. QLoRA and 4bit Quantization, Step 4): one
// launch per pass, every workgroup staging what it reads in LDS with all its
// loads issued at once, fp32 arithmetic with single roundings:
//
//   forward  (26. ..., Step 3):  u = x A^T,  y = fmaf(s, u B^T, x W^^T)
//   backward (22. ..., Step 1):  g = s (dy B),  dB = s (dy^T u),  dA = g^T x,
//                                dx = dy W^ + g A
//
// W^ is dequantised element by element as table[index] * scale (26. ...,
// Step 4).  Each workgroup forms u (and g) itself, 16 lanes per value
// (strided partial sums, then a butterfly over the 16 lanes); every other
// output is one thread's fp32 chain in index order, so tokens with equal
// inputs get bit-identical outputs.
//
// Forward: workgroup b owns outputs n in [64 b, 64 b + 64); thread t takes
// n = 64 b + t % 64 for the tokens m = t / 64 + 4 i.  Backward: workgroup b
// owns the input columns k in [64 b, 64 b + 64) of dx and dA (one
// 64-element chunk of every weight row, staged in LDS) and the rows n in
// [64 b, 64 b + 64) of dB.
#include "kernels.h"

namespace qlora {

constexpr int kTinyThreads = 256;
constexpr int kTinyMaxM = 16;
constexpr int kTinyMaxR = 32;
constexpr int kTinyMaxN = 512;
constexpr int kTinyMaxK = 256;

bool tiny_preferred(int act_dtype, int64_t M, int64_t N, int64_t K, int32_t r) {
  return act_dtype == QL_F32 && M <= kTinyMaxM && r <= kTinyMaxR && N <= kTinyMaxN &&
         K <= kTinyMaxK;
}

// dst[i] = src[i] for i < n (n <= 8192, n % 4 == 0, 16-byte aligned): all loads first
__device__ __forceinline__ void stage_f32(float *dst, const float *__restrict__ src, int n, int t) {
  f32x4 v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int e = 4 * (t + kTinyThreads * i);
    if (e < n) v[i] = *reinterpret_cast<const f32x4 *>(src + e);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int e = 4 * (t + kTinyThreads * i);
    if (e < n) *reinterpret_cast<f32x4 *>(dst + e) = v[i];
  }
}

// sum_c P[c] Q[c * qs] over c < C (C <= CMAX) by a group of 16 lanes: lane
// l16 takes c = l16 + 16 i, Q from global (all its loads first), P from
// LDS; every lane of the group returns the sum
template <int CMAX, typename QT>
__device__ __forceinline__ float dot16(const float *p, const QT *__restrict__ q, int C, int64_t qs,
                                       int l16) {
  float qv[CMAX / 16];
#pragma unroll
  for (int i = 0; i < CMAX / 16; ++i) {
    const int c = l16 + 16 * i;
    qv[i] = c < C ? load_as_f32(q, c * qs) : 0.0f;
  }
  float acc = 0.0f;
#pragma unroll
  for (int i = 0; i < CMAX / 16; ++i) {
    const int c = l16 + 16 * i;
    if (c < C) acc = __builtin_fmaf(p[c], qv[i], acc);
  }
#pragma unroll
  for (int d = 8; d > 0; d >>= 1) acc += __shfl_xor(acc, d, 16);
  return acc;
}

template <typename LT>
__global__ __launch_bounds__(kTinyThreads) void k_tiny_fwd(
    const float *__restrict__ x, int M, const uint8_t *__restrict__ packed, BlockScales sc,
    int N, int K, const LT *__restrict__ A, const LT *__restrict__ B, int32_t r, float s,
    float *__restrict__ y, float *__restrict__ u_save) {
  __shared__ __attribute__((aligned(16))) float xs[kTinyMaxM * kTinyMaxK];
  __shared__ float us[kTinyMaxM][kTinyMaxR];
  __shared__ float cb[16];
  const int t = threadIdx.x;
  const int n = 64 * blockIdx.x + (t & 63);
  const int nc = n < N ? n : N - 1;
  // this thread's weight row (K / 2 <= 256 bytes), its block constants and
  // its row of B, all in flight with the activation staging
  uint32_t wv[kTinyMaxK / 8];
  const uint8_t *wr = packed + ((int64_t)nc * K >> 1);
#pragma unroll
  for (int i = 0; i < kTinyMaxK / 32; ++i)
    if (32 * i < K) {
      const u32x4 v = *reinterpret_cast<const u32x4 *>(wr + 16 * i);
      wv[4 * i] = v[0]; wv[4 * i + 1] = v[1]; wv[4 * i + 2] = v[2]; wv[4 * i + 3] = v[3];
    }
  float wa[kTinyMaxK / 64];
#pragma unroll
  for (int i = 0; i < kTinyMaxK / 64; ++i)
    if (64 * i < K) wa[i] = sc((int64_t)nc * (K / 64) + i);
  float bv[kTinyMaxR];
#pragma unroll
  for (int j = 0; j < kTinyMaxR; ++j)
    if (j < r) bv[j] = load_as_f32(B, (int64_t)nc * r + j);
  if (t < 16) cb[t] = c_nf4[t];
  stage_f32(xs, x, M * K, t);
  __syncthreads();
  // u[m][j]: 16 groups of 16 lanes
  for (int o = t >> 4; o < M * r; o += kTinyThreads / 16) {
    const int m = o / r, j = o % r;
    const float v = dot16<kTinyMaxK>(xs + m * K, A + (int64_t)j * K, K, 1, t & 15);
    if ((t & 15) == 0) {
      us[m][j] = v;
      if (u_save && blockIdx.x == 0) u_save[m * r + j] = v;
    }
  }
  __syncthreads();
  if (n >= N) return;
  for (int m = t >> 6; m < M; m += kTinyThreads / 64) {
    const float *xr = xs + m * K;
    float acc = 0.0f;
#pragma unroll
    for (int i = 0; i < kTinyMaxK / 8; ++i) {
      if (8 * i >= K) break;
      const float a = wa[i >> 3];
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const uint32_t byte = (wv[i] >> (8 * b)) & 0xFFu;
        acc = __builtin_fmaf(xr[8 * i + 2 * b], cb[byte >> 4] * a, acc);
        acc = __builtin_fmaf(xr[8 * i + 2 * b + 1], cb[byte & 15] * a, acc);
      }
    }
    float l = 0.0f;
#pragma unroll
    for (int j = 0; j < kTinyMaxR; ++j)
      if (j < r) l = __builtin_fmaf(us[m][j], bv[j], l);
    y[(int64_t)m * N + n] = __builtin_fmaf(s, l, acc);
  }
}

template <typename LT>
__global__ __launch_bounds__(kTinyThreads) void k_tiny_bwd(
    const float *__restrict__ dy, const float *__restrict__ x, int M,
    const uint8_t *__restrict__ packed, BlockScales sc, int N, int K, const LT *__restrict__ A,
    const LT *__restrict__ B, int32_t r, float s, const float *__restrict__ u_saved,
    float *__restrict__ dx, float *__restrict__ dA, float *__restrict__ dB, int accumulate) {
  __shared__ __attribute__((aligned(16))) float dys[kTinyMaxM * kTinyMaxN];
  __shared__ __attribute__((aligned(16))) float xs[kTinyMaxM * kTinyMaxK];
  __shared__ __attribute__((aligned(16))) uint8_t wk[kTinyMaxN * 32];  // [n][32 bytes]
  __shared__ float wks[kTinyMaxN];
  __shared__ float us[kTinyMaxM][kTinyMaxR];
  __shared__ float gs[kTinyMaxM][kTinyMaxR];
  __shared__ float cb[16];
  const int t = threadIdx.x;
  const int k0 = 64 * blockIdx.x;
  const bool has_k = k0 < K;
  // the workgroup's 64-column chunk of every weight row and its constants
  if (has_k && dx) {
    for (int e = t; e < 2 * N; e += kTinyThreads) {  // two 16-byte pieces per row
      const int nn = e >> 1;
      *reinterpret_cast<u32x4 *>(wk + 32 * nn + 16 * (e & 1)) =
          *reinterpret_cast<const u32x4 *>(packed + (((int64_t)nn * K + k0) >> 1) + 16 * (e & 1));
    }
    for (int nn = t; nn < N; nn += kTinyThreads) wks[nn] = sc((int64_t)nn * (K / 64) + k0 / 64);
  }
  if (t < 16) cb[t] = c_nf4[t];
  stage_f32(dys, dy, M * N, t);
  stage_f32(xs, x, M * K, t);
  __syncthreads();
  // u (given, or x A^T) and g = s (dy B)
  for (int o = t >> 4; o < 2 * M * r; o += kTinyThreads / 16) {
    const int which = o / (M * r), mj = o % (M * r);
    const int m = mj / r, j = mj % r;
    float v;
    if (which == 0)
      v = u_saved ? u_saved[m * r + j]
                  : dot16<kTinyMaxK>(xs + m * K, A + (int64_t)j * K, K, 1, t & 15);
    else
      v = s * dot16<kTinyMaxN>(dys + m * N, B + j, N, r, t & 15);
    if ((t & 15) == 0) {
      if (which == 0) us[m][j] = v;
      else gs[m][j] = v;
    }
  }
  __syncthreads();
  // dB[n][j] = s (sum_m dy[m][n] u[m][j]) for rows n in [64 b, 64 b + 64)
  for (int e = t; e < 64 * r; e += kTinyThreads) {
    const int n = 64 * blockIdx.x + e / r, j = e % r;
    if (n >= N) break;
    float acc = 0.0f;
#pragma unroll 4
    for (int m = 0; m < M; ++m) acc = __builtin_fmaf(dys[m * N + n], us[m][j], acc);
    const float v = s * acc;
    const int64_t o = (int64_t)n * r + j;
    dB[o] = accumulate ? dB[o] + v : v;
  }
  if (!has_k) return;
  // dA[j][k] = sum_m g[m][j] x[m][k] for k in the workgroup's chunk
  for (int e = t; e < 64 * r; e += kTinyThreads) {
    const int j = e >> 6, k = k0 + (e & 63);
    float acc = 0.0f;
#pragma unroll 4
    for (int m = 0; m < M; ++m) acc = __builtin_fmaf(gs[m][j], xs[m * K + k], acc);
    const int64_t o = (int64_t)j * K + k;
    dA[o] = accumulate ? dA[o] + acc : acc;
  }
  if (!dx) return;
  // dx[m][k] = sum_n dy[m][n] W^[n][k] + sum_j g[m][j] A[j][k]
  const int kl = t & 63, k = k0 + kl;
  float av[kTinyMaxR];
#pragma unroll
  for (int j = 0; j < kTinyMaxR; ++j)
    if (j < r) av[j] = load_as_f32(A, (int64_t)j * K + k);
  for (int m = t >> 6; m < M; m += kTinyThreads / 64) {
    const float *dr = dys + m * N;
    float acc = 0.0f;
#pragma unroll 8
    for (int nn = 0; nn < N; ++nn) {
      const uint8_t byte = wk[32 * nn + (kl >> 1)];
      acc = __builtin_fmaf(dr[nn], cb[(kl & 1) ? (byte & 15) : (byte >> 4)] * wks[nn], acc);
    }
    float l = 0.0f;
#pragma unroll
    for (int j = 0; j < kTinyMaxR; ++j)
      if (j < r) l = __builtin_fmaf(gs[m][j], av[j], l);
    dx[(int64_t)m * K + k] = acc + l;
  }
}

int launch_tiny_fwd(const void *x, int64_t M, const uint8_t *packed, BlockScales sc, int64_t N,
                    int64_t K, const void *A, const void *B, int lora_dtype, int32_t r, float s,
                    void *y, float *u_save, hipStream_t stream) {
  const dim3 grid((unsigned)((N + 63) / 64));
  if (lora_dtype == QL_F32)
    hipLaunchKernelGGL(k_tiny_fwd<float>, grid, dim3(kTinyThreads), 0, stream, (const float *)x,
                       (int)M, packed, sc, (int)N, (int)K, (const float *)A, (const float *)B, r,
                       s, (float *)y, u_save);
  else
    hipLaunchKernelGGL(k_tiny_fwd<uint16_t>, grid, dim3(kTinyThreads), 0, stream,
                       (const float *)x, (int)M, packed, sc, (int)N, (int)K, (const uint16_t *)A,
                       (const uint16_t *)B, r, s, (float *)y, u_save);
  QL_HIP_CHECK_LAUNCH();
  return QL_OK;
}

int launch_tiny_bwd(const void *dy, const void *x, int64_t M, const uint8_t *packed,
                    BlockScales sc, int64_t N, int64_t K, const void *A, const void *B,
                    int lora_dtype, int32_t r, float s, const float *u_saved, void *dx, float *dA,
                    float *dB, bool accumulate, hipStream_t stream) {
  const int64_t blocks = (N > K ? N : K);
  const dim3 grid((unsigned)((blocks + 63) / 64));
  if (lora_dtype == QL_F32)
    hipLaunchKernelGGL(k_tiny_bwd<float>, grid, dim3(kTinyThreads), 0, stream,
                       (const float *)dy, (const float *)x, (int)M, packed, sc, (int)N, (int)K,
                       (const float *)A, (const float *)B, r, s, u_saved, (float *)dx, dA, dB,
                       accumulate ? 1 : 0);
  else
    hipLaunchKernelGGL(k_tiny_bwd<uint16_t>, grid, dim3(kTinyThreads), 0, stream,
                       (const float *)dy, (const float *)x, (int)M, packed, sc, (int)N, (int)K,
                       (const uint16_t *)A, (const uint16_t *)B, r, s, u_saved, (float *)dx, dA,
                       dB, accumulate ? 1 : 0);
  QL_HIP_CHECK_LAUNCH();
  return QL_OK;
}

}  // namespace qlora
