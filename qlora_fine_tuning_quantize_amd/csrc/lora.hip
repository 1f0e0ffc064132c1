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
// rows on the matrix cores (16-bit P): v_mfma_f32_16x16x32_{bf16,f16} with
// A = 16 rows of P x 32 contraction values (read straight from global, 16 B
// per lane) and B = the LoRA factor slice staged in LDS in P's format [j][c].
// Wave w of the workgroup owns rows 16w..16w+15 of a 64-row tile and all JT
// 16-wide rank tiles; the workgroup covers one CS-wide slice of the
// contraction in a single round trip, with every trip count fixed at
// compile time: the factor loads are issued first (8 values per load along
// the factor's contiguous dimension, or single values for ranks / shapes
// that are not 8-aligned), then all CS/32 loads of P, then the factor is
// written to LDS (only its loads are waited for), one barrier, the MFMAs,
// and the fp32 partial sums of the slice.  Rows past M and contraction
// positions past C load clamped addresses and use zeros instead.
// Operand layout (gfx950): A lane l holds A[l % 16][8*(l/16) .. +8]; B lane l
// holds B[8*(l/16) .. +8][l % 16]; result lane l holds D[4*(l/16) .. +4][l % 16].
// ---------------------------------------------------------------------------
constexpr int kMRowsTile = 64;

// factor layouts: rows j contiguous in c (Q(j, c) = Q[j * ldq_j + c]), rows c
// contiguous in j (Q(j, c) = Q[c * ldq_c + j]), or element-wise
enum { kQRowJ = 0, kQRowC = 1, kQElem = 2 };

template <typename QT>
constexpr int rows_cs_of(int jt) {
  // bounds the staged factor to 8 (16-bit) or 4 (fp32) 8-value loads per lane
  return (sizeof(QT) == 2 ? 1024 : 512) / jt > 512 ? 512 : (sizeof(QT) == 2 ? 1024 : 512) / jt;
}

static int rows_jt(int32_t r) {
  const int jt = (r + 15) / 16;
  return jt <= 1 ? 1 : jt <= 2 ? 2 : jt <= 4 ? 4 : 8;
}
static int rows_cs(int32_t r, int q_dtype) {
  const int jt = rows_jt(r);
  return q_dtype == QL_F32 ? rows_cs_of<float>(jt) : rows_cs_of<uint16_t>(jt);
}

// 8 consecutive values of a factor row as fp32 (zero where !ok); QT is
// float or a 16-bit storage type
template <typename QT>
struct Vec8 {
  u32x4 w;
  __device__ __forceinline__ void load(const QT *p) { w = *reinterpret_cast<const u32x4 *>(p); }
  __device__ __forceinline__ float get(int e, bool ok) const {
    const uint32_t h = w[e >> 1];
    return ok ? ((e & 1) ? Half<QT>::hi(h) : Half<QT>::lo(h)) : 0.0f;
  }
};
template <>
struct Vec8<float> {
  f32x4 a, b;
  __device__ __forceinline__ void load(const float *p) {
    a = *reinterpret_cast<const f32x4 *>(p);
    b = *reinterpret_cast<const f32x4 *>(p + 4);
  }
  __device__ __forceinline__ float get(int e, bool ok) const {
    return ok ? (e < 4 ? a[e] : b[e - 4]) : 0.0f;
  }
};

// AT: the 16-bit format of P and of the matrix-core operands.  DROP: P is
// the activation x of the LoRA dropout; its dropped elements are zeroed as
// loaded (the 1/(1-p) scale is applied by the reduction).
template <int CS, int JT, typename AT, typename QT, int QMODE, bool DROP>
__global__ __launch_bounds__(256) void k_rows_mfma(const AT *__restrict__ P, int64_t M,
                                                   int64_t C, const QT *__restrict__ Q,
                                                   int64_t ldq_j, int64_t ldq_c, int32_t r,
                                                   float *__restrict__ partial, Dropout dr) {
  constexpr int QST = 2 * CS + 16;   // bytes per staged rank row
  constexpr int JW = JT * 16;
  __shared__ __attribute__((aligned(16))) uint8_t qs[JW * QST];
  const int t = threadIdx.x, wave = t >> 6, lane = t & 63;
  const int li = lane & 15, q = lane >> 4;
  const int64_t c0 = (int64_t)blockIdx.y * CS;

  // ---- factor loads (issued first) ----
  constexpr int NV = JW * CS / 8 / 256;          // 8-value loads per lane
  constexpr int NE = (QMODE == kQElem) ? JW * CS / 256 : 1;
  Vec8<QT> qv[QMODE == kQElem ? 1 : NV];
  float qe[NE];
  if constexpr (QMODE == kQRowJ) {
#pragma unroll
    for (int b = 0; b < NV; ++b) {
      const int e = t + 256 * b, j = e / (CS / 8), c8 = e % (CS / 8);
      const int64_t c = c0 + 8 * c8;
      const int jc = j < r ? j : r - 1;
      const int64_t cc = c + 8 <= C ? c : C - 8;
      qv[b].load(Q + (int64_t)jc * ldq_j + cc);
    }
  } else if constexpr (QMODE == kQRowC) {
#pragma unroll
    for (int b = 0; b < NV; ++b) {
      const int e = t + 256 * b, cc = e / (JW / 8), j8 = e % (JW / 8);
      const int64_t c = c0 + cc < C ? c0 + cc : C - 1;
      const int jc = 8 * j8 + 8 <= r ? 8 * j8 : r - 8;
      qv[b].load(Q + c * ldq_c + jc);
    }
  } else {
#pragma unroll
    for (int b = 0; b < NE; ++b) {
      const int e = t + 256 * b;
      int j, cc;
      if (ldq_c == 1) { j = e / CS; cc = e % CS; } else { cc = e / JW; j = e % JW; }
      const int64_t c = c0 + cc;
      qe[b] = (j < r && c < C) ? load_as_f32(Q, j * ldq_j + c * ldq_c) : 0.0f;
    }
  }

  // ---- P loads: row mrow, contraction c0 + 32 i + 8 q ----
  const int64_t mrow = (int64_t)blockIdx.x * kMRowsTile + 16 * wave + li;
  const AT *prow = P + (mrow < M ? mrow : M - 1) * C;
  u32x4 a[CS / 32];
#pragma unroll
  for (int i = 0; i < CS / 32; ++i) {
    const int64_t c = c0 + 32 * i + 8 * q;
    a[i] = *reinterpret_cast<const u32x4 *>(prow + (c + 8 <= C ? c : C - 8));
    if (c + 8 > C) a[i] = u32x4{0u, 0u, 0u, 0u};
  }
  if constexpr (DROP) {  // after every load is out; C % 8 == 0 on this path
#pragma unroll
    for (int i = 0; i < CS / 32; ++i) {
      const int64_t c = c0 + 32 * i + 8 * q;
      if (c + 8 <= C) a[i] = dropout_mask8(dr, (uint64_t)mrow * C + c, a[i]);
    }
  }

  // ---- factor slice to LDS, 16-bit [j][c] ----
  if constexpr (QMODE == kQRowJ) {
#pragma unroll
    for (int b = 0; b < NV; ++b) {
      const int e = t + 256 * b, j = e / (CS / 8), c8 = e % (CS / 8);
      const bool ok = j < r && c0 + 8 * c8 + 8 <= C;
      *reinterpret_cast<u32x4 *>(qs + j * QST + 16 * c8) =
          u32x4{Half<AT>::pack2(qv[b].get(0, ok), qv[b].get(1, ok)),
                Half<AT>::pack2(qv[b].get(2, ok), qv[b].get(3, ok)),
                Half<AT>::pack2(qv[b].get(4, ok), qv[b].get(5, ok)),
                Half<AT>::pack2(qv[b].get(6, ok), qv[b].get(7, ok))};
    }
  } else if constexpr (QMODE == kQRowC) {
#pragma unroll
    for (int b = 0; b < NV; ++b) {
      const int e = t + 256 * b, cc = e / (JW / 8), j8 = e % (JW / 8);
      const bool ok = c0 + cc < C && 8 * j8 + 8 <= r;
#pragma unroll
      for (int jj = 0; jj < 8; ++jj)
        *reinterpret_cast<uint16_t *>(qs + (8 * j8 + jj) * QST + 2 * cc) =
            Half<AT>::bits(qv[b].get(jj, ok));
    }
  } else {
#pragma unroll
    for (int b = 0; b < NE; ++b) {
      const int e = t + 256 * b;
      int j, cc;
      if (ldq_c == 1) { j = e / CS; cc = e % CS; } else { cc = e / JW; j = e % JW; }
      *reinterpret_cast<uint16_t *>(qs + j * QST + 2 * cc) = Half<AT>::bits(qe[b]);
    }
  }
  __syncthreads();

  f32x4 acc[JT];
#pragma unroll
  for (int i = 0; i < JT; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < CS / 32; ++i) {
#pragma unroll
    for (int jt = 0; jt < JT; ++jt) {
      const u32x4 b = *reinterpret_cast<const u32x4 *>(qs + (16 * jt + li) * QST +
                                                       2 * (32 * i + 8 * q));
      acc[jt] = Half<AT>::mfma16(a[i], b, acc[jt]);
    }
  }
  const int64_t mbase = (int64_t)blockIdx.x * kMRowsTile + 16 * wave + 4 * q;
#pragma unroll
  for (int jt = 0; jt < JT; ++jt) {
    const int j = 16 * jt + li;
    if (j >= r) continue;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int64_t m = mbase + v;
      if (m < M) partial[((int64_t)blockIdx.y * M + m) * r + j] = acc[jt][v];
    }
  }
}

// out[e] = scale * sum_s partial[s][e], s in increasing order (8 slices per
// batch are loaded before they are added).
__global__ __launch_bounds__(256) void k_reduce_slices(const float *__restrict__ partial, int S,
                                                       int64_t count, float scale,
                                                       float *__restrict__ out) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= count) return;
  float s = 0.0f;
  for (int i0 = 0; i0 < S; i0 += 8) {
    float v[8];
#pragma unroll
    for (int b = 0; b < 8; ++b) v[b] = i0 + b < S ? partial[(int64_t)(i0 + b) * count + e] : 0.0f;
#pragma unroll
    for (int b = 0; b < 8; ++b)
      if (i0 + b < S) s += v[b];
  }
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

// Slices of the matrix-core rows kernel: one per CS-wide piece of the
// contraction (the partial buffer is sized for the fp32-factor case, which
// has the narrower slices).
static int mrows_slices(int64_t C, int32_t r, int q_dtype) {
  return (int)((C + rows_cs(r, q_dtype) - 1) / rows_cs(r, q_dtype));
}

static bool rows_use_mfma(int p_dtype, int64_t C) { return p_dtype != QL_F32 && C % 8 == 0; }

size_t lora_rows_partial_floats(int64_t M, int64_t C, int32_t r) {
  const int64_t s1 = rows_slices(M, C), s2 = mrows_slices(C, r, QL_F32);
  return (size_t)(s1 > s2 ? s1 : s2) * (size_t)M * (size_t)r;
}

int launch_lora_rows_ws(const void *P, int p_dtype, int64_t M, int64_t C, const void *Q,
                        int q_dtype, int64_t ldq_j, int64_t ldq_c, int32_t r, float scale,
                        float *out, float *partial, hipStream_t stream, int *slices,
                        const Dropout *drop) {
  if (M <= 0) return QL_OK;
  int S;
  if (drop && (!rows_use_mfma(p_dtype, C) || ldq_c != 1 || ldq_j % 8 != 0 || C < 8))
    return QL_EUNSUPPORTED;
  const Dropout dr = drop ? *drop : Dropout{0u, 0u, 0u};
  if (rows_use_mfma(p_dtype, C)) {
    S = mrows_slices(C, r, q_dtype);
    const dim3 grid((unsigned)((M + kMRowsTile - 1) / kMRowsTile), (unsigned)S);
    const int jt = rows_jt(r);
    // 8-value loads need the loaded factor rows 8-aligned (the factor base
    // pointer is 16-byte aligned) and at least 8 long
    int mode = kQElem;
    if (ldq_c == 1 && C % 8 == 0 && ldq_j % 8 == 0 && C >= 8) mode = kQRowJ;
    else if (ldq_j == 1 && r % 8 == 0 && ldq_c % 8 == 0) mode = kQRowC;
#define QL_ROWS_M(JTV, QT, MODEV, DRV)                                                           \
  hipLaunchKernelGGL((k_rows_mfma<rows_cs_of<QT>(JTV), JTV, AT, QT, MODEV, DRV>), grid,          \
                     dim3(256), 0, stream, (const AT *)P, M, C, (const QT *)Q, ldq_j, ldq_c, r,  \
                     partial, dr)
#define QL_ROWS_Q(JTV, QT)                                                                       \
  do {                                                                                           \
    if (drop) QL_ROWS_M(JTV, QT, kQRowJ, true);                                                  \
    else if (mode == kQRowJ) QL_ROWS_M(JTV, QT, kQRowJ, false);                                  \
    else if (mode == kQRowC) QL_ROWS_M(JTV, QT, kQRowC, false);                                  \
    else QL_ROWS_M(JTV, QT, kQElem, false);                                                      \
  } while (0)
#define QL_ROWS_JT(JTV) \
  do { if (q_dtype == QL_F32) QL_ROWS_Q(JTV, float); else QL_ROWS_Q(JTV, AT); } while (0)
    // a 16-bit factor has the activations' format (checked by the caller)
    with_half(p_dtype, [&](auto *tag) {
      using AT = elem_of<decltype(tag)>;
      if (jt == 1) QL_ROWS_JT(1);
      else if (jt == 2) QL_ROWS_JT(2);
      else if (jt == 4) QL_ROWS_JT(4);
      else QL_ROWS_JT(8);
    });
#undef QL_ROWS_JT
#undef QL_ROWS_Q
#undef QL_ROWS_M
  } else {
    S = rows_slices(M, C);
    int64_t slice = (C + S - 1) / S;
    slice = (slice + kRowsChunk - 1) / kRowsChunk * kRowsChunk;
    const dim3 grid((unsigned)((M + kRowsTM - 1) / kRowsTM), (unsigned)S);
    with_type(p_dtype, [&](auto *pt) {
      with_type(q_dtype, [&](auto *qt) {
        hipLaunchKernelGGL((k_lora_rows<elem_of<decltype(pt)>, elem_of<decltype(qt)>>), grid,
                           dim3(256), 0, stream, P, M, C, Q, ldq_j, ldq_c, r, slice, partial);
      });
    });
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
// cols on the matrix cores (16-bit P): D[j][c] = sum_m R^T[j][m] P[m][c] with
// v_mfma_f32_16x16x32_{bf16,f16}.  The workgroup owns 64 columns (wave w: columns
// 16w..16w+15, all JT rank tiles) and one TM-token slice, in one round trip
// with compile-time trip counts: the loads of R (fp32, 4 ranks per load when
// r % 4 == 0) and of the P tile (16 bytes per lane) are all issued first,
// then R^T is written to LDS in P's format [j][m] and the P tile as [m][c]
// (128-byte rows), one barrier, the MFMAs, and the fp32 partial sums.  The
// B operand (8 consecutive tokens of one column) comes from gfx950's
// transposing LDS read: for a group of 16 lanes naming rows m0..m0+3
// (lanes 4e..4e+3 -> row m0+e, four columns each), output lane i receives
// column i of those rows.  Within a row the four 32-byte column groups are
// rotated by a row-dependent amount, so the 8 rows one read pass touches
// (and the 2 rows one 16-lane store pass touches) hit distinct banks.
// ---------------------------------------------------------------------------
constexpr int kMColsTile = 64;
constexpr int kMColsTM = 256;  // tokens per workgroup

typedef short s16x4 __attribute__((ext_vector_type(4)));

// byte offset of 16-byte piece h (columns 8h..8h+7) of staged token row m
__device__ __forceinline__ int ps_off(int m, int h) {
  const int pcg = ((h >> 1) + (m >> 1) + 2 * ((m >> 3) & 1)) & 3;
  return m * 128 + ((2 * pcg + (h & 1)) << 4);
}

__device__ __forceinline__ u32x2 lds_tr16(const uint8_t *p) {
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4 *)(p));
  return __builtin_bit_cast(u32x2, v);
}

// AT: the 16-bit format of P and of the matrix-core operands.  DROP: P is
// the activation x of the LoRA dropout; its dropped elements are zeroed as
// loaded (the 1/(1-p) scale is applied by the reduction).
// ColsOut: with a single token slice (gridDim.y == 1) the workgroup writes
// the finished result itself, with the arithmetic of k_reduce_cols for one
// slice (out = scale * (0 + sum), or out += that, [r][C] or transposed);
// otherwise out is NULL and the slice's partial sums go to `partial`.
struct ColsOut {
  float *out;
  float scale;
  int c_major, accumulate;
};

template <int TM, int JT, typename AT, bool RVEC, bool DROP>
__global__ __launch_bounds__(256) void k_cols_mfma(const float *__restrict__ R, int64_t M,
                                                   int32_t r, const AT *__restrict__ P,
                                                   int64_t C, float *__restrict__ partial,
                                                   Dropout dr, ColsOut co) {
  constexpr int JW = JT * 16;
  constexpr int RST = 2 * TM + 16;  // bytes per staged rank row
  __shared__ __attribute__((aligned(16))) uint8_t ps[TM * 128];
  __shared__ __attribute__((aligned(16))) uint8_t rs[JW * RST];
  const int t = threadIdx.x, wave = t >> 6, lane = t & 63;
  const int li = lane & 15, q = lane >> 4;
  const int64_t ct0 = (int64_t)blockIdx.x * kMColsTile;
  const int64_t m0 = (int64_t)blockIdx.y * TM;

  // ---- R loads: rows m0 .. m0 + TM, ranks 0 .. JW ----
  constexpr int NR = RVEC ? TM * JW / 4 / 256 : TM * JW / 256;
  f32x4 rv[RVEC ? NR : 1];
  float re[RVEC ? 1 : NR];
  if constexpr (RVEC) {
#pragma unroll
    for (int b = 0; b < NR; ++b) {
      const int e = t + 256 * b, mm = e / (JW / 4), j4 = e % (JW / 4);
      const int64_t m = m0 + mm < M ? m0 + mm : M - 1;
      const int jc = 4 * j4 + 4 <= r ? 4 * j4 : r - 4;
      rv[b] = *reinterpret_cast<const f32x4 *>(R + m * r + jc);
    }
  } else {
#pragma unroll
    for (int b = 0; b < NR; ++b) {
      const int e = t + 256 * b, mm = e / JW, j = e % JW;
      re[b] = (m0 + mm < M && j < r) ? R[(m0 + mm) * r + j] : 0.0f;
    }
  }
  // ---- P tile loads: rows (t >> 3) + 32 i, piece t & 7 ----
  const int prow = t >> 3, ph = t & 7;
  const int64_t pc = ct0 + 8 * ph;
  const bool cok = pc + 8 <= C;
  u32x4 pv[TM / 32];
#pragma unroll
  for (int i = 0; i < TM / 32; ++i) {
    const int64_t m = m0 + prow + 32 * i;
    pv[i] = *reinterpret_cast<const u32x4 *>(P + (m < M ? m : M - 1) * C + (cok ? pc : C - 8));
    if (m >= M || !cok) pv[i] = u32x4{0u, 0u, 0u, 0u};
  }
  if constexpr (DROP) {  // after every load is out; C % 8 == 0 on this path
#pragma unroll
    for (int i = 0; i < TM / 32; ++i) {
      const int64_t m = m0 + prow + 32 * i;
      if (m < M && cok) pv[i] = dropout_mask8(dr, (uint64_t)m * C + pc, pv[i]);
    }
  }
  // ---- to LDS ----
  if constexpr (RVEC) {
#pragma unroll
    for (int b = 0; b < NR; ++b) {
      const int e = t + 256 * b, mm = e / (JW / 4), j4 = e % (JW / 4);
      const bool ok = m0 + mm < M && 4 * j4 + 4 <= r;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)
        *reinterpret_cast<uint16_t *>(rs + (4 * j4 + jj) * RST + 2 * mm) =
            Half<AT>::bits(ok ? rv[b][jj] : 0.0f);
    }
  } else {
#pragma unroll
    for (int b = 0; b < NR; ++b) {
      const int e = t + 256 * b, mm = e / JW, j = e % JW;
      *reinterpret_cast<uint16_t *>(rs + j * RST + 2 * mm) = Half<AT>::bits(re[b]);
    }
  }
#pragma unroll
  for (int i = 0; i < TM / 32; ++i)
    *reinterpret_cast<u32x4 *>(ps + ps_off(prow + 32 * i, ph)) = pv[i];
  __syncthreads();

  f32x4 acc[JT];
#pragma unroll
  for (int i = 0; i < JT; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  // transposing-read supplier address: rows 8q + (li >> 2) (+4), columns
  // 16 wave + 4 (li & 3)
  const int tr_col = 16 * wave + 4 * (li & 3);
  const int tr_h = tr_col >> 3, tr_b = 2 * (tr_col & 7);
#pragma unroll
  for (int kk = 0; kk < TM; kk += 32) {
    const int row = kk + 8 * q + (li >> 2);
    const u32x2 lo = lds_tr16(ps + ps_off(row, tr_h) + tr_b);
    const u32x2 hi = lds_tr16(ps + ps_off(row + 4, tr_h) + tr_b);
    const u32x4 b = u32x4{lo[0], lo[1], hi[0], hi[1]};
#pragma unroll
    for (int jt = 0; jt < JT; ++jt) {
      const u32x4 a =
          *reinterpret_cast<const u32x4 *>(rs + (16 * jt + li) * RST + 2 * (kk + 8 * q));
      acc[jt] = Half<AT>::mfma16(a, b, acc[jt]);
    }
  }
  const int64_t c = ct0 + 16 * wave + li;
  if (c < C) {
#pragma unroll
    for (int jt = 0; jt < JT; ++jt) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int j = 16 * jt + 4 * q + v;
        if (j >= r) continue;
        if (co.out) {
#pragma clang fp contract(off)
          const float sum = 0.0f + acc[jt][v];  // k_reduce_cols' sum over one slice
          const int64_t o = co.c_major ? c * r + j : (int64_t)j * C + c;
          co.out[o] = co.accumulate ? co.out[o] + co.scale * sum : co.scale * sum;
        } else {
          partial[((int64_t)blockIdx.y * r + j) * C + c] = acc[jt][v];
        }
      }
    }
  }
}

// out = scale * sum_s partial[s][j][c] (s in increasing order, 8 slices per
// batch loaded before they are added); written as [r][C] or transposed [C][r],
// or added to what out holds (accumulate != 0, one fp32 addition).  One
// launch serves one or two such sums (jobs a and b, b empty when b.S == 0):
// blocks [0, blocks(a)) take a, the rest b.
__device__ __forceinline__ void reduce_cols_one(const ColsReduce &jb, int64_t e) {
  // accumulation is the product scale * s, rounded, then one addition
#pragma clang fp contract(off)
  const int64_t count = (int64_t)jb.r * jb.C;
  if (e >= count) return;
  float s = 0.0f;
  for (int i0 = 0; i0 < jb.S; i0 += 8) {
    float v[8];
#pragma unroll
    for (int b = 0; b < 8; ++b)
      v[b] = i0 + b < jb.S ? jb.partial[(int64_t)(i0 + b) * count + e] : 0.0f;
#pragma unroll
    for (int b = 0; b < 8; ++b)
      if (i0 + b < jb.S) s += v[b];
  }
  const int64_t j = e / jb.C, c = e % jb.C;
  const int64_t o = jb.c_major ? c * jb.r + j : e;
  jb.out[o] = jb.accumulate ? jb.out[o] + jb.scale * s : jb.scale * s;
}

static int64_t reduce_cols_blocks(const ColsReduce &jb) {
  return jb.S > 0 ? ((int64_t)jb.r * jb.C + 255) / 256 : 0;
}

__global__ __launch_bounds__(256) void k_reduce_cols(ColsReduce a, ColsReduce b, int64_t blocks_a) {
  const int64_t blk = blockIdx.x;
  if (blk < blocks_a) reduce_cols_one(a, blk * 256 + threadIdx.x);
  else reduce_cols_one(b, (blk - blocks_a) * 256 + threadIdx.x);
}

int launch_reduce_cols(const ColsReduce &a, const ColsReduce &b, hipStream_t stream) {
  const int64_t na = reduce_cols_blocks(a), nb = reduce_cols_blocks(b);
  if (na + nb == 0) return QL_OK;
  hipLaunchKernelGGL(k_reduce_cols, dim3((unsigned)(na + nb)), dim3(256), 0, stream, a, b, na);
  QL_HIP_CHECK_LAUNCH();
  return QL_OK;
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

// Token slices of the matrix-core cols kernel: one per TM tokens.
static int mcols_slices(int64_t M) { return (int)((M + kMColsTM - 1) / kMColsTM); }

static bool cols_use_mfma(int p_dtype, int64_t C) { return p_dtype != QL_F32 && C % 8 == 0; }

size_t lora_cols_partial_floats(int64_t M, int64_t C, int32_t r) {
  const int64_t s1 = cols_slices(M, C), s2 = mcols_slices(M);
  return (size_t)(s1 > s2 ? s1 : s2) * (size_t)r * (size_t)C;
}

int launch_lora_cols(const float *R, int64_t M, int32_t r, const void *P, int p_dtype, int64_t C,
                     float scale, bool out_c_major, float *out, float *partial,
                     hipStream_t stream, bool accumulate, const Dropout *drop,
                     ColsReduce *pending) {
  if (pending) pending->S = 0;
  if (C <= 0) return QL_OK;
  int S;
  if (drop && !cols_use_mfma(p_dtype, C)) return QL_EUNSUPPORTED;
  const Dropout dr = drop ? *drop : Dropout{0u, 0u, 0u};
  if (cols_use_mfma(p_dtype, C)) {
    S = mcols_slices(M);
    const dim3 grid((unsigned)((C + kMColsTile - 1) / kMColsTile), (unsigned)S);
    // one token slice: the kernel writes the result, no reduction launch
    const ColsOut co{S == 1 ? out : nullptr, scale, out_c_major ? 1 : 0, accumulate ? 1 : 0};
    const bool rvec = r % 4 == 0;
#define QL_COLS_M(JTV, RV, DRV)                                                               \
  hipLaunchKernelGGL((k_cols_mfma<kMColsTM, JTV, AT, RV, DRV>), grid, dim3(256), 0, stream, R, \
                     M, r, (const AT *)P, C, partial, dr, co)
#define QL_COLS_JT(JTV)                                                                          \
  do {                                                                                           \
    if (rvec) { if (drop) QL_COLS_M(JTV, true, true); else QL_COLS_M(JTV, true, false); }        \
    else { if (drop) QL_COLS_M(JTV, false, true); else QL_COLS_M(JTV, false, false); }           \
  } while (0)
    const int jt = rows_jt(r);
    with_half(p_dtype, [&](auto *tag) {
      using AT = elem_of<decltype(tag)>;
      if (jt == 1) QL_COLS_JT(1);
      else if (jt == 2) QL_COLS_JT(2);
      else if (jt == 4) QL_COLS_JT(4);
      else QL_COLS_JT(8);
    });
#undef QL_COLS_JT
#undef QL_COLS_M
    QL_HIP_CHECK_LAUNCH();
    if (S == 1) return QL_OK;
  } else {
    S = cols_slices(M, C);
    const int64_t slice = (M + S - 1) / S;
    const dim3 grid((unsigned)((C + kColsTC - 1) / kColsTC), (unsigned)S);
    with_type(p_dtype, [&](auto *pt) {
      hipLaunchKernelGGL((k_lora_cols<elem_of<decltype(pt)>>), grid, dim3(256), 0, stream, R, M,
                         r, P, C, slice, partial);
    });
  }
  QL_HIP_CHECK_LAUNCH();
  const ColsReduce job{partial, S, r, C, scale, out_c_major ? 1 : 0, accumulate ? 1 : 0, out};
  if (pending) {  // the caller launches it, possibly together with another
    *pending = job;
    return QL_OK;
  }
  return launch_reduce_cols(job, ColsReduce{nullptr, 0, 0, 0, 0.0f, 0, 0, nullptr}, stream);
}

}  // namespace qlora
