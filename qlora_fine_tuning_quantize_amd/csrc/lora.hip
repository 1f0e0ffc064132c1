// lora.hip -- the rank-r products of the LoRA bypass (26. QLoRA and 4bit
// Quantization, Step 3: y = x W^T + (x A^T) B^T * alpha/r; the backward of
// that formula gives g = s dy B, dB = s dy^T u, dA = g^T x).
//
// All are skinny: one dimension is the rank r <= 128, the contraction runs
// over K, N or the token count M.  They split the contraction across
// workgroups and reduce the fp32 partial sums in a second, fixed-order pass,
// so results are deterministic run to run.
#include "kernels.h"

namespace qlora {

template <typename T>
__device__ __forceinline__ float ld(const void *p, int64_t i) {
  return load_as_f32(reinterpret_cast<const T *>(p), i);
}

// ---------------------------------------------------------------------------
// rows: partial[s][m][j] = sum_{c in slice s} P[m][c] * Q(j, c)
// 256 lanes, 32 rows of P per workgroup, contraction chunks of 64 staged in
// LDS as fp32; lane (m = t % 32, j0 = t / 32) owns outputs j = j0 + 8 i.
// ---------------------------------------------------------------------------
constexpr int kRowsTM = 32;
constexpr int kRowsChunk = 64;

template <typename PT, typename QT>
__global__ __launch_bounds__(256) void k_lora_rows(const void *__restrict__ P, int64_t M, int64_t C,
                                                   const void *__restrict__ Q, int64_t ldq_j,
                                                   int64_t ldq_c, int32_t r, int64_t slice,
                                                   float *__restrict__ partial) {
  __shared__ float ps[kRowsTM][kRowsChunk + 1];
  __shared__ float qs[128][kRowsChunk + 1];
  const int t = threadIdx.x;
  const int64_t m0 = (int64_t)blockIdx.x * kRowsTM;
  const int64_t c_begin = (int64_t)blockIdx.y * slice;
  const int64_t c_end = c_begin + slice < C ? c_begin + slice : C;
  const int ml = t % kRowsTM, j0 = t / kRowsTM;
  float acc[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.0f;
  for (int64_t c0 = c_begin; c0 < c_end; c0 += kRowsChunk) {
    for (int e = t; e < kRowsTM * kRowsChunk; e += 256) {
      const int rr = e / kRowsChunk, cc = e % kRowsChunk;
      const int64_t m = m0 + rr, c = c0 + cc;
      ps[rr][cc] = (m < M && c < c_end) ? ld<PT>(P, m * C + c) : 0.0f;
    }
    for (int e = t; e < r * kRowsChunk; e += 256) {
      const int jj = e / kRowsChunk, cc = e % kRowsChunk;
      const int64_t c = c0 + cc;
      qs[jj][cc] = (c < c_end) ? ld<QT>(Q, jj * ldq_j + c * ldq_c) : 0.0f;
    }
    __syncthreads();
    for (int cc = 0; cc < kRowsChunk; ++cc) {
      const float pv = ps[ml][cc];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int j = j0 + 8 * i;
        if (j < r) acc[i] = __builtin_fmaf(pv, qs[j][cc], acc[i]);
      }
    }
    __syncthreads();
  }
  const int64_t m = m0 + ml;
  if (m < M) {
    float *dst = partial + ((int64_t)blockIdx.y * M + m) * r;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int j = j0 + 8 * i;
      if (j < r) dst[j] = acc[i];
    }
  }
}

// out[e] = scale * sum_s partial[s][e], s in increasing order.
__global__ __launch_bounds__(256) void k_reduce_slices(const float *__restrict__ partial, int S,
                                                       int64_t count, float scale,
                                                       float *__restrict__ out) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= count) return;
  float s = 0.0f;
  for (int i = 0; i < S; ++i) s += partial[(int64_t)i * count + e];
  out[e] = scale * s;
}

static int rows_slices(int64_t M, int64_t C) {
  const int64_t mt = (M + kRowsTM - 1) / kRowsTM;
  int64_t s = 512 / mt;
  const int64_t max_s = (C + kRowsChunk - 1) / kRowsChunk;
  if (s > max_s) s = max_s;
  if (s > 64) s = 64;
  if (s < 1) s = 1;
  return (int)s;
}

size_t lora_rows_partial_floats(int64_t M, int64_t C, int32_t r) {
  return (size_t)rows_slices(M, C) * (size_t)M * (size_t)r;
}

int launch_lora_rows_ws(const void *P, int p_dtype, int64_t M, int64_t C, const void *Q,
                        int q_dtype, int64_t ldq_j, int64_t ldq_c, int32_t r, float scale,
                        float *out, float *partial, hipStream_t stream) {
  if (M <= 0) return QL_OK;
  const int S = rows_slices(M, C);
  int64_t slice = (C + S - 1) / S;
  slice = (slice + kRowsChunk - 1) / kRowsChunk * kRowsChunk;
  const dim3 grid((unsigned)((M + kRowsTM - 1) / kRowsTM), (unsigned)S);
#define QL_ROWS(PT, QT)                                                                        \
  hipLaunchKernelGGL((k_lora_rows<PT, QT>), grid, dim3(256), 0, stream, P, M, C, Q, ldq_j,   \
                     ldq_c, r, slice, partial)
  if (p_dtype == QL_BF16 && q_dtype == QL_BF16) QL_ROWS(uint16_t, uint16_t);
  else if (p_dtype == QL_BF16) QL_ROWS(uint16_t, float);
  else if (q_dtype == QL_BF16) QL_ROWS(float, uint16_t);
  else QL_ROWS(float, float);
#undef QL_ROWS
  QL_HIP_CHECK_LAUNCH();
  const int64_t count = M * r;
  hipLaunchKernelGGL(k_reduce_slices, dim3((unsigned)((count + 255) / 256)), dim3(256), 0, stream,
                     partial, S, count, scale, out);
  QL_HIP_CHECK_LAUNCH();
  return QL_OK;
}

// ---------------------------------------------------------------------------
// cols: partial[s][j][c] = sum_{m in slice s} R[m][j] * P[m][c]
// 64 columns per workgroup; lane (c = t % 64, j0 = t / 64) owns j = j0 + 4 i.
// R rows are staged through LDS 64 at a time.
// ---------------------------------------------------------------------------
constexpr int kColsTC = 64;
constexpr int kColsChunk = 64;

template <typename PT>
__global__ __launch_bounds__(256) void k_lora_cols(const float *__restrict__ R, int64_t M,
                                                   int32_t r, const void *__restrict__ P,
                                                   int64_t C, int64_t slice,
                                                   float *__restrict__ partial) {
  __shared__ float rs[kColsChunk][129];
  const int t = threadIdx.x;
  const int cl = t % kColsTC, j0 = t / kColsTC;
  const int64_t c = (int64_t)blockIdx.x * kColsTC + cl;
  const int64_t m_begin = (int64_t)blockIdx.y * slice;
  const int64_t m_end = m_begin + slice < M ? m_begin + slice : M;
  float acc[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) acc[i] = 0.0f;
  for (int64_t mc = m_begin; mc < m_end; mc += kColsChunk) {
    for (int e = t; e < kColsChunk * r; e += 256) {
      const int mm = e / r, jj = e % r;
      const int64_t m = mc + mm;
      rs[mm][jj] = (m < m_end) ? R[m * r + jj] : 0.0f;
    }
    __syncthreads();
    const int n_in = (int)((m_end - mc) < kColsChunk ? (m_end - mc) : kColsChunk);
    for (int mm = 0; mm < n_in; ++mm) {
      const float pv = (c < C) ? ld<PT>(P, (mc + mm) * C + c) : 0.0f;
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        const int j = j0 + 4 * i;
        if (j < r) acc[i] = __builtin_fmaf(rs[mm][j], pv, acc[i]);
      }
    }
    __syncthreads();
  }
  if (c < C) {
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const int j = j0 + 4 * i;
      if (j < r) partial[((int64_t)blockIdx.y * r + j) * C + c] = acc[i];
    }
  }
}

// out = scale * sum_s partial[s][j][c]; written as [r][C] or transposed [C][r].
__global__ __launch_bounds__(256) void k_reduce_cols(const float *__restrict__ partial, int S,
                                                     int32_t r, int64_t C, float scale,
                                                     int c_major, float *__restrict__ out) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t count = (int64_t)r * C;
  if (e >= count) return;
  float s = 0.0f;
  for (int i = 0; i < S; ++i) s += partial[(int64_t)i * count + e];
  const int64_t j = e / C, c = e % C;
  if (c_major)
    out[c * r + j] = scale * s;
  else
    out[e] = scale * s;
}

static int cols_slices(int64_t M, int64_t C) {
  const int64_t ct = (C + kColsTC - 1) / kColsTC;
  int64_t s = 1024 / ct;
  const int64_t max_s = (M + kColsChunk - 1) / kColsChunk;
  if (s > max_s) s = max_s;
  if (s > 32) s = 32;
  if (s < 1) s = 1;
  return (int)s;
}

size_t lora_cols_partial_floats(int64_t M, int64_t C, int32_t r) {
  return (size_t)cols_slices(M, C) * (size_t)r * (size_t)C;
}

int launch_lora_cols(const float *R, int64_t M, int32_t r, const void *P, int p_dtype, int64_t C,
                     float scale, bool out_c_major, float *out, float *partial,
                     hipStream_t stream) {
  if (C <= 0) return QL_OK;
  const int S = cols_slices(M, C);
  int64_t slice = (M + S - 1) / S;
  const dim3 grid((unsigned)((C + kColsTC - 1) / kColsTC), (unsigned)S);
  if (p_dtype == QL_BF16)
    hipLaunchKernelGGL(k_lora_cols<uint16_t>, grid, dim3(256), 0, stream, R, M, r, P, C, slice,
                       partial);
  else
    hipLaunchKernelGGL(k_lora_cols<float>, grid, dim3(256), 0, stream, R, M, r, P, C, slice,
                       partial);
  QL_HIP_CHECK_LAUNCH();
  const int64_t count = (int64_t)r * C;
  hipLaunchKernelGGL(k_reduce_cols, dim3((unsigned)((count + 255) / 256)), dim3(256), 0, stream,
                     partial, S, r, C, scale, out_c_major ? 1 : 0, out);
  QL_HIP_CHECK_LAUNCH();
  return QL_OK;
}

}  // namespace qlora
