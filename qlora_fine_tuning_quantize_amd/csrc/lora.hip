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

// ---------------------------------------------------------------------------
// rows on the matrix cores (bf16 P): v_mfma_f32_16x16x32_bf16 with
// A = 16 rows of P x 32 contraction values (read straight from global, 16 B
// per lane) and B = the LoRA factor staged in LDS as bf16 [j][c].  Wave w of
// the workgroup owns rows 16w..16w+15 of a 64-row tile and every 16-wide
// rank tile; the workgroup covers one slice of the contraction.
// Operand layout (gfx950): A lane l holds A[l % 16][8*(l/16) .. +8]; B lane l
// holds B[8*(l/16) .. +8][l % 16]; result lane l holds D[4*(l/16) .. +4][l % 16].
// ---------------------------------------------------------------------------
constexpr int kMRowsTile = 64;
constexpr int kMRowsChunk = 256;
constexpr int kQsStride = kMRowsChunk * 2 + 16;  // bytes per staged rank row (bank-shifted)

template <typename QT>
__global__ __launch_bounds__(256) void k_rows_mfma(const uint16_t *__restrict__ P, int64_t M,
                                                   int64_t C, const QT *__restrict__ Q,
                                                   int64_t ldq_j, int64_t ldq_c, int32_t r,
                                                   int64_t slice, float *__restrict__ partial) {
  __shared__ __attribute__((aligned(16))) uint8_t qs[128 * kQsStride];
  const int t = threadIdx.x, wave = t >> 6, lane = t & 63;
  const int li = lane & 15, q = lane >> 4;
  const int JT = (r + 15) >> 4;
  const int64_t mrow = (int64_t)blockIdx.x * kMRowsTile + 16 * wave + li;
  const int64_t cb = (int64_t)blockIdx.y * slice;
  const int64_t ce = cb + slice < C ? cb + slice : C;
  f32x4 acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  const uint16_t *prow = P + mrow * C;
  for (int64_t c0 = cb; c0 < ce; c0 += kMRowsChunk) {
    for (int e = t; e < JT * 16 * kMRowsChunk; e += 256) {
      const int j = e / kMRowsChunk, cc = e % kMRowsChunk;
      const int64_t c = c0 + cc;
      const float v = (j < r && c < ce) ? load_as_f32(Q, j * ldq_j + c * ldq_c) : 0.0f;
      *reinterpret_cast<uint16_t *>(qs + j * kQsStride + 2 * cc) = f32_to_bf16_bits(v);
    }
    __syncthreads();
    // all eight 16-byte loads of the chunk in flight before the matrix ops
    u32x4 a[kMRowsChunk / 32];
#pragma unroll
    for (int i = 0; i < kMRowsChunk / 32; ++i) {
      const int64_t c = c0 + 32 * i + 8 * q;
      a[i] = u32x4{0u, 0u, 0u, 0u};
      if (mrow < M && c + 8 <= ce) a[i] = *reinterpret_cast<const u32x4 *>(prow + c);
    }
#pragma unroll
    for (int i = 0; i < kMRowsChunk / 32; ++i) {
#pragma unroll 1
      for (int jt = 0; jt < JT; ++jt) {
        const u32x4 b = *reinterpret_cast<const u32x4 *>(qs + (16 * jt + li) * kQsStride +
                                                         2 * (32 * i + 8 * q));
        acc[jt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a[i]),
                                                          __builtin_bit_cast(bf16x8, b), acc[jt],
                                                          0, 0, 0);
      }
    }
    __syncthreads();
  }
  const int64_t mbase = (int64_t)blockIdx.x * kMRowsTile + 16 * wave + 4 * q;
#pragma unroll
  for (int jt = 0; jt < 8; ++jt) {
    const int j = 16 * jt + li;
    if (jt >= JT || j >= r) continue;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int64_t m = mbase + v;
      if (m < M) partial[((int64_t)blockIdx.y * M + m) * r + j] = acc[jt][v];
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

// Slices of the matrix-core rows kernel: about 512 workgroups, slices a
// multiple of the 256-wide LDS chunk.
static int mrows_slices(int64_t M, int64_t C) {
  const int64_t mt = (M + kMRowsTile - 1) / kMRowsTile;
  int64_t s = 512 / mt;
  const int64_t max_s = (C + kMRowsChunk - 1) / kMRowsChunk;
  if (s > max_s) s = max_s;
  if (s < 1) s = 1;
  return (int)s;
}

static bool rows_use_mfma(int p_dtype, int64_t C) { return p_dtype == QL_BF16 && C % 8 == 0; }

size_t lora_rows_partial_floats(int64_t M, int64_t C, int32_t r) {
  const int64_t s1 = rows_slices(M, C), s2 = mrows_slices(M, C);
  return (size_t)(s1 > s2 ? s1 : s2) * (size_t)M * (size_t)r;
}

int launch_lora_rows_ws(const void *P, int p_dtype, int64_t M, int64_t C, const void *Q,
                        int q_dtype, int64_t ldq_j, int64_t ldq_c, int32_t r, float scale,
                        float *out, float *partial, hipStream_t stream, int *slices) {
  if (M <= 0) return QL_OK;
  int S;
  if (rows_use_mfma(p_dtype, C)) {
    S = mrows_slices(M, C);
    int64_t slice = (C + S - 1) / S;
    slice = (slice + kMRowsChunk - 1) / kMRowsChunk * kMRowsChunk;
    const dim3 grid((unsigned)((M + kMRowsTile - 1) / kMRowsTile), (unsigned)S);
    if (q_dtype == QL_BF16)
      hipLaunchKernelGGL(k_rows_mfma<uint16_t>, grid, dim3(256), 0, stream, (const uint16_t *)P, M,
                         C, (const uint16_t *)Q, ldq_j, ldq_c, r, slice, partial);
    else
      hipLaunchKernelGGL(k_rows_mfma<float>, grid, dim3(256), 0, stream, (const uint16_t *)P, M, C,
                         (const float *)Q, ldq_j, ldq_c, r, slice, partial);
  } else {
    S = rows_slices(M, C);
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
  }
  QL_HIP_CHECK_LAUNCH();
  if (slices) *slices = S;
  if (!out) return QL_OK;
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

// ---------------------------------------------------------------------------
// cols on the matrix cores (bf16 P): D[j][c] = sum_m R^T[j][m] P[m][c] with
// v_mfma_f32_16x16x32_bf16.  Per 64-token chunk the workgroup stages its
// 64 x 64 tile of P in LDS ([m][c], 132-byte rows so that the column reads
// below spread over all banks) and R^T as bf16 [j][m].  Wave w owns columns
// 16w..16w+15 of the tile and every rank tile; its B operand (8 consecutive
// tokens of one column) is gathered from LDS 16 bits at a time.
// ---------------------------------------------------------------------------
constexpr int kMColsTile = 64;
constexpr int kMColsChunk = 64;
constexpr int kPsStride = 132;                   // bytes per staged token row
constexpr int kRsStride = kMColsChunk * 2 + 16;  // bytes per staged rank row

__global__ __launch_bounds__(256) void k_cols_mfma(const float *__restrict__ R, int64_t M,
                                                   int32_t r, const uint16_t *__restrict__ P,
                                                   int64_t C, int64_t slice,
                                                   float *__restrict__ partial) {
  __shared__ __attribute__((aligned(16))) uint8_t ps[kMColsChunk * kPsStride];
  __shared__ __attribute__((aligned(16))) uint8_t rs[128 * kRsStride];
  const int t = threadIdx.x, wave = t >> 6, lane = t & 63;
  const int li = lane & 15, q = lane >> 4;
  const int JT = (r + 15) >> 4;
  const int64_t ct0 = (int64_t)blockIdx.x * kMColsTile;
  const int64_t mb = (int64_t)blockIdx.y * slice;
  const int64_t me = mb + slice < M ? mb + slice : M;
  f32x4 acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int col = 16 * wave + li;
  for (int64_t mc = mb; mc < me; mc += kMColsChunk) {
    // P tile: 64 rows x 8 chunks of 16 B; stored as 4-byte words (132-byte rows)
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int id = t + 256 * i;
      const int row = id >> 3, ch = id & 7;
      const int64_t m = mc + row, c = ct0 + 8 * ch;
      u32x4 v = u32x4{0u, 0u, 0u, 0u};
      if (m < me && c + 8 <= C) v = *reinterpret_cast<const u32x4 *>(P + m * C + c);
      uint32_t *dst = reinterpret_cast<uint32_t *>(ps + row * kPsStride + 16 * ch);
      dst[0] = v.x;
      dst[1] = v.y;
      dst[2] = v.z;
      dst[3] = v.w;
    }
    for (int e = t; e < JT * 16 * kMColsChunk; e += 256) {
      const int j = e / kMColsChunk, mm = e % kMColsChunk;
      const int64_t m = mc + mm;
      const float v = (j < r && m < me) ? R[m * r + j] : 0.0f;
      *reinterpret_cast<uint16_t *>(rs + j * kRsStride + 2 * mm) = f32_to_bf16_bits(v);
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < kMColsChunk; kk += 32) {
      uint32_t bw[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t lo = *reinterpret_cast<const uint16_t *>(ps + (kk + 8 * q + 2 * e) * kPsStride + 2 * col);
        const uint32_t hi = *reinterpret_cast<const uint16_t *>(ps + (kk + 8 * q + 2 * e + 1) * kPsStride + 2 * col);
        bw[e] = lo | (hi << 16);
      }
      const u32x4 b = u32x4{bw[0], bw[1], bw[2], bw[3]};
#pragma unroll
      for (int jt = 0; jt < 8; ++jt) {
        if (jt < JT) {
          const u32x4 a =
              *reinterpret_cast<const u32x4 *>(rs + (16 * jt + li) * kRsStride + 2 * (kk + 8 * q));
          acc[jt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                            __builtin_bit_cast(bf16x8, b), acc[jt],
                                                            0, 0, 0);
        }
      }
    }
    __syncthreads();
  }
  const int64_t c = ct0 + col;
  if (c < C) {
#pragma unroll
    for (int jt = 0; jt < 8; ++jt) {
      if (jt >= JT) continue;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int j = 16 * jt + 4 * q + v;
        if (j < r) partial[((int64_t)blockIdx.y * r + j) * C + c] = acc[jt][v];
      }
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

static int mcols_slices(int64_t M, int64_t C) {
  const int64_t ct = (C + kMColsTile - 1) / kMColsTile;
  int64_t s = 768 / ct;
  const int64_t max_s = (M + kMColsChunk - 1) / kMColsChunk;
  if (s > max_s) s = max_s;
  if (s < 1) s = 1;
  return (int)s;
}

static bool cols_use_mfma(int p_dtype, int64_t C) { return p_dtype == QL_BF16 && C % 8 == 0; }

size_t lora_cols_partial_floats(int64_t M, int64_t C, int32_t r) {
  const int64_t s1 = cols_slices(M, C), s2 = mcols_slices(M, C);
  return (size_t)(s1 > s2 ? s1 : s2) * (size_t)r * (size_t)C;
}

int launch_lora_cols(const float *R, int64_t M, int32_t r, const void *P, int p_dtype, int64_t C,
                     float scale, bool out_c_major, float *out, float *partial,
                     hipStream_t stream) {
  if (C <= 0) return QL_OK;
  int S;
  if (cols_use_mfma(p_dtype, C)) {
    S = mcols_slices(M, C);
    int64_t slice = (M + S - 1) / S;
    slice = (slice + kMColsChunk - 1) / kMColsChunk * kMColsChunk;
    const dim3 grid((unsigned)((C + kMColsTile - 1) / kMColsTile), (unsigned)S);
    hipLaunchKernelGGL(k_cols_mfma, grid, dim3(256), 0, stream, R, M, r, (const uint16_t *)P, C,
                       slice, partial);
  } else {
    S = cols_slices(M, C);
    const int64_t slice = (M + S - 1) / S;
    const dim3 grid((unsigned)((C + kColsTC - 1) / kColsTC), (unsigned)S);
    if (p_dtype == QL_BF16)
      hipLaunchKernelGGL(k_lora_cols<uint16_t>, grid, dim3(256), 0, stream, R, M, r, P, C, slice,
                         partial);
    else
      hipLaunchKernelGGL(k_lora_cols<float>, grid, dim3(256), 0, stream, R, M, r, P, C, slice,
                         partial);
  }
  QL_HIP_CHECK_LAUNCH();
  const int64_t count = (int64_t)r * C;
  hipLaunchKernelGGL(k_reduce_cols, dim3((unsigned)((count + 255) / 256)), dim3(256), 0, stream,
                     partial, S, r, C, scale, out_c_major ? 1 : 0, out);
  QL_HIP_CHECK_LAUNCH();
  return QL_OK;
}

}  // namespace qlora
