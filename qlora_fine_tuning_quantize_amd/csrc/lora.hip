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

// DROP: P is the activation x of the LoRA dropout; dropped elements are
// staged as zeros (the reduction applies 1/(1-p)).
template <typename PT, typename QT, bool DROP>
__global__ __launch_bounds__(256) void k_lora_rows(const void *__restrict__ P, int64_t M, int64_t C,
                                                   const void *__restrict__ Q, int64_t ldq_j,
                                                   int64_t ldq_c, int32_t r, int64_t slice,
                                                   float *__restrict__ partial, Dropout dr) {
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
      const bool in = m < M && c < c_end;
      ps[rr][cc] = in && (!DROP || dropout_keep1(dr, (uint64_t)(m * C + c))) ? ld<PT>(P, m * C + c)
                                                                             : 0.0f;
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
// 16-wide rank tiles; the workgroup covers nsub consecutive CS-wide chunks
// of the contraction (one slice), chunk after chunk, with every per-chunk
// trip count fixed at compile time: the factor loads are issued first (8
// values per load along the factor's contiguous dimension, or single values
// for ranks / shapes that are not 8-aligned), then all CS/32 loads of P, then
// the factor is written to LDS (only its loads are waited for), one barrier,
// the MFMAs; the slice's fp32 sums are written once at the end.  Rows past M
// and contraction positions past C load clamped addresses and use zeros
// instead.
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
                                                   float *__restrict__ partial, Dropout dr,
                                                   int nsub) {
  constexpr int QST = 2 * CS + 16;   // bytes per staged rank row
  constexpr int JW = JT * 16;
  __shared__ __attribute__((aligned(16))) uint8_t qs[JW * QST];
  const int t = threadIdx.x, wave = t >> 6, lane = t & 63;
  const int li = lane & 15, q = lane >> 4;
  const int64_t cs0 = (int64_t)blockIdx.y * CS * nsub;
  constexpr int NV = JW * CS / 8 / 256;          // 8-value loads per lane
  constexpr int NE = (QMODE == kQElem) ? JW * CS / 256 : 1;

  f32x4 acc[JT];
#pragma unroll
  for (int i = 0; i < JT; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  // kQRowC (factor rows c contiguous in j, r % 8 == 0): a thread loads NV
  // consecutive rows c of one 8-rank group and stages them transposed, as 8
  // rank rows of NV 16-bit values (one 8- or 16-byte LDS store each).  Thread
  // bits 0-2: low c block, bit 3: low rank group, the rest the high parts, so
  // that one 16-lane store pass covers 16 distinct bank quads.
  constexpr int NCB = CS / NV;                    // c blocks
  static_assert(QMODE != kQRowC || (NCB % 8 == 0 && (JW / 8) % 2 == 0 &&
                                    NCB * (JW / 8) == 256 && (NV == 4 || NV == 8)),
                "factor blocks tile the chunk");
  auto rowc_block = [&](int tt, int &cb, int &j8) {
    const int hi = tt >> 4;
    cb = (tt & 7) + 8 * (hi % (NCB / 8));
    j8 = ((tt >> 3) & 1) + 2 * (hi / (NCB / 8));
  };
  // One CS-wide chunk from c0 into acc.  Per-thread indices come from tt, a
  // copy of the thread index the compiler may not assume constant across
  // chunks, so addresses are recomputed per chunk rather than held in
  // registers over the loop.
  auto chunk = [&](int tt, int64_t c0, bool after) {
    const int w = tt >> 6, l = tt & 63, lj = l & 15, lq = l >> 4;
    // ---- factor loads (issued first) ----
    Vec8<QT> qv[QMODE == kQElem ? 1 : NV];
    float qe[NE];
    if constexpr (QMODE == kQRowJ) {
#pragma unroll
      for (int b = 0; b < NV; ++b) {
        const int e = tt + 256 * b, j = e / (CS / 8), c8 = e % (CS / 8);
        const int64_t c = c0 + 8 * c8;
        const int jc = j < r ? j : r - 1;
        const int64_t cc = c + 8 <= C ? c : C - 8;
        qv[b].load(Q + (int64_t)jc * ldq_j + cc);
      }
    } else if constexpr (QMODE == kQRowC) {
      int cb, j8;
      rowc_block(tt, cb, j8);
      const QT *qb = Q + c0 * ldq_c;  // uniform
      const int jc = 8 * j8 + 8 <= r ? 8 * j8 : r - 8;
      const int clast = (int)(C - 1 - c0);
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        const int cr = NV * cb + i;
        qv[i].load(qb + (int64_t)(cr < clast ? cr : clast) * ldq_c + jc);
      }
    } else {
#pragma unroll
      for (int b = 0; b < NE; ++b) {
        const int e = tt + 256 * b;
        int j, cc;
        if (ldq_c == 1) { j = e / CS; cc = e % CS; } else { cc = e / JW; j = e % JW; }
        const int64_t c = c0 + cc;
        qe[b] = (j < r && c < C) ? load_as_f32(Q, j * ldq_j + c * ldq_c) : 0.0f;
      }
    }

    // ---- P loads: row mrow, contraction c0 + 32 i + 8 lq (32-bit offsets
    // from the tile's uniform base: 64 C < 2^31 on this path) ----
    const int64_t mt0 = (int64_t)blockIdx.x * kMRowsTile;
    const int mr = 16 * w + lj;
    const int mrc = mt0 + mr < M ? mr : (int)(M - 1 - mt0);
    const AT *pb = P + mt0 * C + c0;  // uniform
    u32x4 a[CS / 32];
#pragma unroll
    for (int i = 0; i < CS / 32; ++i) {
      const int64_t c = c0 + 32 * i + 8 * lq;
      const int cl = c + 8 <= C ? 32 * i + 8 * lq : (int)(C - 8 - c0);
      a[i] = *reinterpret_cast<const u32x4 *>(reinterpret_cast<const uint8_t *>(pb) +
                                               (uint32_t)((mrc * (int)C + cl) * 2));
    }

    if (after) __syncthreads();  // the previous chunk's factor has been read
    // ---- factor chunk to LDS, 16-bit [j][c] ----
    if constexpr (QMODE == kQRowJ) {
#pragma unroll
      for (int b = 0; b < NV; ++b) {
        const int e = tt + 256 * b, j = e / (CS / 8), c8 = e % (CS / 8);
        const bool ok = j < r && c0 + 8 * c8 + 8 <= C;
        u32x4 v;
        if constexpr (sizeof(QT) == 2) {  // the operands' own format: copied
          v = ok ? qv[b].w : u32x4{0u, 0u, 0u, 0u};
        } else {
          v = u32x4{Half<AT>::pack2(qv[b].get(0, ok), qv[b].get(1, ok)),
                    Half<AT>::pack2(qv[b].get(2, ok), qv[b].get(3, ok)),
                    Half<AT>::pack2(qv[b].get(4, ok), qv[b].get(5, ok)),
                    Half<AT>::pack2(qv[b].get(6, ok), qv[b].get(7, ok))};
        }
        *reinterpret_cast<u32x4 *>(qs + j * QST + 16 * c8) = v;
      }
    } else if constexpr (QMODE == kQRowC) {
      int cb, j8;
      rowc_block(tt, cb, j8);
      const bool jok = 8 * j8 + 8 <= r;
      bool ok[NV];
#pragma unroll
      for (int i = 0; i < NV; ++i) ok[i] = jok && c0 + NV * cb + i < C;
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        uint32_t o[NV / 2];
#pragma unroll
        for (int k = 0; k < NV / 2; ++k) {
          if constexpr (sizeof(QT) == 2) {
            // halves jj of rows 2k (low) and 2k + 1 (high), by byte select
            const uint32_t lo = ok[2 * k] ? qv[2 * k].w[jj >> 1] : 0u;
            const uint32_t hi = ok[2 * k + 1] ? qv[2 * k + 1].w[jj >> 1] : 0u;
            o[k] = __builtin_amdgcn_perm(hi, lo, (jj & 1) ? 0x07060302u : 0x05040100u);
          } else {
            o[k] = Half<AT>::pack2(qv[2 * k].get(jj, ok[2 * k]),
                                   qv[2 * k + 1].get(jj, ok[2 * k + 1]));
          }
        }
        uint8_t *dst = qs + (8 * j8 + jj) * QST + 2 * NV * cb;
        if constexpr (NV == 8)
          *reinterpret_cast<u32x4 *>(dst) = u32x4{o[0], o[1], o[2], o[3]};
        else
          *reinterpret_cast<u32x2 *>(dst) = u32x2{o[0], o[1]};
      }
    } else {
#pragma unroll
      for (int b = 0; b < NE; ++b) {
        const int e = tt + 256 * b;
        int j, cc;
        if (ldq_c == 1) { j = e / CS; cc = e % CS; } else { cc = e / JW; j = e % JW; }
        *reinterpret_cast<uint16_t *>(qs + j * QST + 2 * cc) = Half<AT>::bits(qe[b]);
      }
    }
    __syncthreads();
    // P pieces past C zeroed, dropout applied: where the operands are used
    // (no earlier wait on the P loads)
#pragma unroll
    for (int i = 0; i < CS / 32; ++i) {
      const int64_t c = c0 + 32 * i + 8 * lq;
      if (c + 8 > C) a[i] = u32x4{0u, 0u, 0u, 0u};
      else if constexpr (DROP)  // C % 8 == 0 on this path
        a[i] = dropout_mask8(dr, (uint64_t)(mt0 + mr) * C + c, a[i]);
    }
#pragma unroll
    for (int i = 0; i < CS / 32; ++i) {
#pragma unroll
      for (int jt = 0; jt < JT; ++jt) {
        const u32x4 b = *reinterpret_cast<const u32x4 *>(qs + (16 * jt + lj) * QST +
                                                         2 * (32 * i + 8 * lq));
        acc[jt] = Half<AT>::mfma16(a[i], b, acc[jt]);
      }
    }
  };
#pragma unroll 1
  for (int sub = 0; sub < nsub; ++sub) {
    const int64_t c0 = cs0 + (int64_t)sub * CS;
    if (c0 >= C) break;  // uniform
    int tt = t;
    asm volatile("" : "+v"(tt));
    chunk(tt, c0, sub > 0);
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

// Slices of the matrix-core rows kernel: runs of nsub CS-wide chunks of the
// contraction, so that the workgroups (64-row tiles x slices) number about
// 1024; fewer slices write fewer partials (M x r floats each).
struct MRowsPlan {
  int S, nsub;
};
static MRowsPlan mrows_plan(int64_t M, int64_t C, int32_t r, int q_dtype) {
  const int64_t cs = rows_cs(r, q_dtype);
  const int64_t chunks = (C + cs - 1) / cs;
  const int64_t tiles = (M + kMRowsTile - 1) / kMRowsTile;
  int64_t S = (1024 + tiles - 1) / tiles;
  if (S > chunks) S = chunks;
  if (S < 1) S = 1;
  MRowsPlan p;
  p.nsub = (int)((chunks + S - 1) / S);
  p.S = (int)((chunks + p.nsub - 1) / p.nsub);
  return p;
}

// 32-bit offsets within a 64-row tile: C < 2^24
static bool rows_use_mfma(int p_dtype, int64_t C) {
  return p_dtype != QL_F32 && C % 8 == 0 && C < ((int64_t)1 << 24);
}

size_t lora_rows_partial_floats(int64_t M, int64_t C, int32_t r) {
  const int64_t s1 = rows_slices(M, C);
  const int64_t sa = mrows_plan(M, C, r, QL_F32).S, sb = mrows_plan(M, C, r, QL_BF16).S;
  const int64_t s2 = sa > sb ? sa : sb;
  return (size_t)(s1 > s2 ? s1 : s2) * (size_t)M * (size_t)r;
}

int launch_lora_rows_ws(const void *P, int p_dtype, int64_t M, int64_t C, const void *Q,
                        int q_dtype, int64_t ldq_j, int64_t ldq_c, int32_t r, float scale,
                        float *out, float *partial, hipStream_t stream, int *slices,
                        const Dropout *drop) {
  if (M <= 0) return QL_OK;
  int S;
  const Dropout dr = drop ? *drop : Dropout{0u, 0u, 0u};
  // the matrix-core kernel masks factor-row-major slices only
  if (rows_use_mfma(p_dtype, C) && (!drop || (ldq_c == 1 && ldq_j % 8 == 0 && C >= 8))) {
    const MRowsPlan mp = mrows_plan(M, C, r, q_dtype);
    S = mp.S;
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
                     partial, dr, mp.nsub)
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
        using PT = elem_of<decltype(pt)>;
        using QT = elem_of<decltype(qt)>;
        if (drop)
          hipLaunchKernelGGL((k_lora_rows<PT, QT, true>), grid, dim3(256), 0, stream, P, M, C, Q,
                             ldq_j, ldq_c, r, slice, partial, dr);
        else
          hipLaunchKernelGGL((k_lora_rows<PT, QT, false>), grid, dim3(256), 0, stream, P, M, C, Q,
                             ldq_j, ldq_c, r, slice, partial, dr);
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

// DROP: as for k_lora_rows.
template <typename PT, bool DROP>
__global__ __launch_bounds__(256) void k_lora_cols(const float *__restrict__ R, int64_t M,
                                                   int32_t r, const void *__restrict__ P,
                                                   int64_t C, int64_t slice,
                                                   float *__restrict__ partial, Dropout dr) {
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
      const int64_t e = (mc + mm) * C + c;
      const float pv = c < C && (!DROP || dropout_keep1(dr, (uint64_t)e)) ? ld<PT>(P, e) : 0.0f;
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
// 16w..16w+15, all JT rank tiles) and one token slice of nsub runs of TM
// tokens.  Per run, with compile-time trip counts: the loads of R (fp32, 4
// ranks per load when r % 4 == 0) and of the P tile (16 bytes per lane) are
// issued together, then R^T is written to LDS in P's format [j][m] and the P
// tile as [m][c] (128-byte rows), one barrier, the next run's loads, the
// MFMAs; the fp32 sums of the slice are written at the end.  The
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

// One product R^T P of a launch: its operands, output, token runs per
// workgroup (nsub) and column tiles; its workgroups are tiles x slices, the
// column tile fastest.
struct ColsJob {
  const float *R;
  const void *P;
  int64_t C;
  float *partial;
  ColsOut co;
  int nsub;
  int64_t tiles;
};

// grid.x = blocks_a + the workgroups of job b (none when b is empty): the
// first blocks_a workgroups take job a, the rest job b.  Both jobs share M,
// r and the dropout of the launch.
template <int TM, int JT, typename AT, bool RVEC, bool DROP>
__global__ __launch_bounds__(256) void k_cols_mfma(ColsJob ja, ColsJob jb, int64_t blocks_a,
                                                   int64_t M, int32_t r, Dropout dr) {
  constexpr int JW = JT * 16;
  constexpr int RST = 2 * TM + 16;  // bytes per staged rank row
  __shared__ __attribute__((aligned(16))) uint8_t ps[TM * 128];
  __shared__ __attribute__((aligned(16))) uint8_t rs[JW * RST];
  const bool second = (int64_t)blockIdx.x >= blocks_a;  // uniform
  const ColsJob &job = second ? jb : ja;
  const float *__restrict__ R = job.R;
  const AT *__restrict__ P = static_cast<const AT *>(job.P);
  const int64_t C = job.C;
  float *__restrict__ partial = job.partial;
  const ColsOut co = job.co;
  const int nsub = job.nsub;
  const int64_t blk = second ? (int64_t)blockIdx.x - blocks_a : (int64_t)blockIdx.x;
  const int64_t bx = blk % job.tiles, by = blk / job.tiles;
  const int t = threadIdx.x, wave = t >> 6, lane = t & 63;
  const int li = lane & 15, q = lane >> 4;
  const int64_t ct0 = bx * kMColsTile;
  // the workgroup's token slice: nsub runs of TM tokens, one after another
  const int64_t ms0 = by * TM * nsub;

  // R with r % 4 == 0 (RVEC): load group g of a thread covers TG consecutive
  // tokens x 4 ranks (TG loads of 16 bytes) and is staged as 4 rank rows of
  // TG 16-bit values (one 8- or 16-byte LDS store each).  Group id
  // gid = tt + 256 g splits as: bits 0-1 the low rank group, bits 2-3 the low
  // token group, the rest (rank group high, token group high), so that the 16
  // lanes of one store pass write 16 distinct bank quads and one load
  // instruction reads whole 64-byte row pieces.  Other r: one value per load.
  constexpr int RG = JW / 4;                      // 4-rank groups
  constexpr int NRV = TM * JW / 4 / 256;          // 16-byte R loads per thread
  constexpr int TG = NRV < 8 ? NRV : 8;           // tokens per load group
  constexpr int NG = NRV / TG;                    // load groups per thread
  static_assert(NG * TG == NRV && (TM / TG) * RG == 256 * NG && RG % 4 == 0,
                "R load groups tile the run");
  constexpr int NR = RVEC ? NRV : TM * JW / 256;
  constexpr int RQ = JW;  // scalar path: threads per R row
  constexpr int RROWS = 256 / RQ;
  static_assert(256 % RQ == 0, "R rows split evenly over the threads");
  f32x4 acc[JT];
#pragma unroll
  for (int i = 0; i < JT; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  // A run of TM tokens: load (R and P to registers), stage (to LDS), mma
  // (into acc).  The next run's loads are issued right after a run is staged,
  // so they are in flight during its matrix ops and barriers.  Per-thread
  // indices come from tt, a copy of the thread index that the compiler may
  // not assume constant across runs: addresses are recomputed per run instead
  // of held in registers over the loop.  Offsets within a run are 32-bit
  // (TM * C < 2^31 on this path).
  f32x4 rv[RVEC ? NRV : 1];
  float re[RVEC ? 1 : NR];
  u32x4 pv[TM / 32];
  auto load = [&](int tt, int64_t m0) {
    const bool full = m0 + TM <= M;  // uniform
    const int mlast = full ? TM - 1 : (int)(M - 1 - m0);  // last row of the run
    const float *Rb = R + m0 * r;
    // P tile: rows prow + 32 i, 8-column piece ph
    const int prow = tt >> 3, ph = tt & 7;
    const int64_t pc = ct0 + 8 * ph;
    const bool cok = pc + 8 <= C;
    const AT *Pb = P + m0 * C + ct0;  // uniform
    const int pcl = cok ? 8 * ph : (int)(C - 8 - ct0);
    if constexpr (RVEC) {
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        const int gid = tt + 256 * g, hi = gid >> 4;
        const int rgi = (gid & 3) + 4 * (hi % (RG / 4));
        const int tgi = ((gid >> 2) & 3) + 4 * (hi / (RG / 4));
        const int col = 4 * rgi + 4 <= r ? 4 * rgi : r - 4;
#pragma unroll
        for (int i = 0; i < TG; ++i) {
          const int row = TG * tgi + i;
          rv[TG * g + i] = *reinterpret_cast<const f32x4 *>(
              reinterpret_cast<const uint8_t *>(Rb) +
              (uint32_t)(((row < mlast ? row : mlast) * r + col) * 4));
        }
      }
    } else {
      const int rm0 = tt / RQ, rl = tt % RQ;
#pragma unroll
      for (int b = 0; b < NR; ++b) {
        const int row = rm0 + RROWS * b;
        re[b] = rl < r && row <= mlast ? Rb[row * r + rl] : 0.0f;
      }
    }
#pragma unroll
    for (int i = 0; i < TM / 32; ++i) {
      const int row = prow + 32 * i;
      const int rc = row < mlast ? row : mlast;
      pv[i] = *reinterpret_cast<const u32x4 *>(reinterpret_cast<const uint8_t *>(Pb) +
                                                (uint32_t)((rc * (int)C + pcl) * 2));
    }
  };
  auto stage = [&](int tt, int64_t m0) {
    const bool full = m0 + TM <= M;  // uniform
    const int mlast = full ? TM - 1 : (int)(M - 1 - m0);
    const int prow = tt >> 3, ph = tt & 7;
    const int64_t pc = ct0 + 8 * ph;
    const bool cok = pc + 8 <= C;
    // ---- to LDS (R and P rows past M, R ranks past r and P pieces past C
    // zeroed) ----
#pragma unroll
    for (int i = 0; i < TM / 32; ++i) {
      const int row = prow + 32 * i;
      if (row > mlast || !cok) pv[i] = u32x4{0u, 0u, 0u, 0u};
      else if constexpr (DROP)  // C % 8 == 0 on this path
        pv[i] = dropout_mask8(dr, (uint64_t)(m0 + row) * C + pc, pv[i]);
    }
    if constexpr (RVEC) {
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        const int gid = tt + 256 * g, hi = gid >> 4;
        const int rgi = (gid & 3) + 4 * (hi % (RG / 4));
        const int tgi = ((gid >> 2) & 3) + 4 * (hi / (RG / 4));
        const bool rok = 4 * rgi + 4 <= r;
        float v[TG][4];
#pragma unroll
        for (int i = 0; i < TG; ++i) {
          const bool ok = rok && TG * tgi + i <= mlast;
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) v[i][jj] = ok ? rv[TG * g + i][jj] : 0.0f;
        }
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          uint8_t *dst = rs + (4 * rgi + jj) * RST + 2 * TG * tgi;
          if constexpr (TG == 8)
            *reinterpret_cast<u32x4 *>(dst) =
                u32x4{Half<AT>::pack2(v[0][jj], v[1][jj]), Half<AT>::pack2(v[2][jj], v[3][jj]),
                      Half<AT>::pack2(v[4][jj], v[5][jj]), Half<AT>::pack2(v[6][jj], v[7][jj])};
          else
            *reinterpret_cast<u32x2 *>(dst) =
                u32x2{Half<AT>::pack2(v[0][jj], v[1][jj]), Half<AT>::pack2(v[2][jj], v[3][jj])};
        }
      }
    } else {
      const int rm0 = tt / RQ, rl = tt % RQ;
#pragma unroll
      for (int b = 0; b < NR; ++b)
        *reinterpret_cast<uint16_t *>(rs + rl * RST + 2 * (rm0 + RROWS * b)) =
            Half<AT>::bits(re[b]);
    }
#pragma unroll
    for (int i = 0; i < TM / 32; ++i)
      *reinterpret_cast<u32x4 *>(ps + ps_off(prow + 32 * i, ph)) = pv[i];
  };
  auto mma = [&](int tt) {
    // ---- acc[jt] += R^T P over the run; transposing-read supplier address:
    // rows 8 q + (li >> 2) (+4), columns 16 wave + 4 (li & 3) ----
    const int w = tt >> 6, l = tt & 63, lj = l & 15, lq = l >> 4;
    const int tr_col = 16 * w + 4 * (lj & 3);
    const int tr_h = tr_col >> 3, tr_b = 2 * (tr_col & 7);
#pragma unroll
    for (int kk = 0; kk < TM; kk += 32) {
      const int row = kk + 8 * lq + (lj >> 2);
      const u32x2 lo = lds_tr16(ps + ps_off(row, tr_h) + tr_b);
      const u32x2 hi = lds_tr16(ps + ps_off(row + 4, tr_h) + tr_b);
      const u32x4 bb = u32x4{lo[0], lo[1], hi[0], hi[1]};
#pragma unroll
      for (int jt = 0; jt < JT; ++jt) {
        const u32x4 a =
            *reinterpret_cast<const u32x4 *>(rs + (16 * jt + lj) * RST + 2 * (kk + 8 * lq));
        acc[jt] = Half<AT>::mfma16(a, bb, acc[jt]);
      }
    }
  };
  const int nrun = (int)((M - ms0 + TM - 1) / TM < nsub ? (M - ms0 + TM - 1) / TM : nsub);
  {
    int tt = t;
    asm volatile("" : "+v"(tt));
    load(tt, ms0);
  }
#pragma unroll 1
  for (int sub = 0; sub < nrun; ++sub) {
    const int64_t m0 = ms0 + (int64_t)sub * TM;
    int tt = t;
    asm volatile("" : "+v"(tt));
    if (sub > 0) __syncthreads();  // the previous run's operands have been read
    stage(tt, m0);
    __syncthreads();
    if (sub + 1 < nrun) load(tt, m0 + TM);
    mma(tt);
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
          partial[(by * r + j) * C + c] = acc[jt][v];
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
  jb.out[e] = jb.accumulate ? jb.out[e] + jb.scale * s : jb.scale * s;
}

// The transposed ([C][r]) result: a workgroup takes 64 columns x 32 ranks;
// each thread sums 8 elements (as above, slices in increasing order, four
// slices of all 8 elements loaded before they are added) into an LDS tile
// [j][c], which is then written with j fastest (128-byte row pieces).
constexpr int kRedTC = 64, kRedTJ = 32;
__device__ __forceinline__ void reduce_cols_tile(const ColsReduce &jb, int64_t blk,
                                                 float (*tile)[kRedTC + 1]) {
#pragma clang fp contract(off)
  constexpr int NE = kRedTC * kRedTJ / 256;
  const int t = threadIdx.x, cl = t % kRedTC, jq = t / kRedTC;
  const int64_t count = (int64_t)jb.r * jb.C;
  const int64_t jtiles = (jb.r + kRedTJ - 1) / kRedTJ;
  const int64_t c0 = blk / jtiles * kRedTC, c = c0 + cl;
  const int j0 = (int)(blk % jtiles) * kRedTJ;
  float s[NE];
#pragma unroll
  for (int k = 0; k < NE; ++k) s[k] = 0.0f;
  for (int i0 = 0; i0 < jb.S; i0 += 4) {
    float v[NE][4];
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int k = 0; k < NE; ++k) {
        const int j = j0 + jq + (256 / kRedTC) * k;
        v[k][b] = i0 + b < jb.S && j < jb.r && c < jb.C
                      ? jb.partial[(int64_t)(i0 + b) * count + (int64_t)j * jb.C + c]
                      : 0.0f;
      }
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int k = 0; k < NE; ++k)
        if (i0 + b < jb.S) s[k] += v[k][b];
  }
#pragma unroll
  for (int k = 0; k < NE; ++k) tile[jq + (256 / kRedTC) * k][cl] = jb.scale * s[k];
  __syncthreads();
  const int ncol = (int)(jb.C - c0 < kRedTC ? jb.C - c0 : kRedTC);
  const int nj = jb.r - j0 < kRedTJ ? jb.r - j0 : kRedTJ;
#pragma unroll
  for (int k = 0; k < NE; ++k) {
    const int idx = t + 256 * k, cc = idx / kRedTJ, jj = idx % kRedTJ;
    if (cc < ncol && jj < nj) {
      const int64_t o = (c0 + cc) * jb.r + j0 + jj;
      const float v = tile[jj][cc];
      jb.out[o] = jb.accumulate ? jb.out[o] + v : v;
    }
  }
}

static int64_t reduce_cols_blocks(const ColsReduce &jb) {
  if (jb.S <= 0) return 0;
  return jb.c_major ? (jb.C + kRedTC - 1) / kRedTC * ((jb.r + kRedTJ - 1) / kRedTJ)
                    : ((int64_t)jb.r * jb.C + 255) / 256;
}

__global__ __launch_bounds__(256) void k_reduce_cols(ColsReduce a, ColsReduce b, int64_t blocks_a) {
  __shared__ float tile[kRedTJ][kRedTC + 1];
  const int64_t blk = blockIdx.x;
  const ColsReduce &jb = blk < blocks_a ? a : b;
  const int64_t bi = blk < blocks_a ? blk : blk - blocks_a;
  if (jb.c_major) reduce_cols_tile(jb, bi, tile);  // uniform
  else reduce_cols_one(jb, bi * 256 + threadIdx.x);
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

// Token slices of the matrix-core cols kernel: runs of TM tokens, nsub runs
// per workgroup, so that the workgroups (column tiles x slices) number about
// 1024: fewer slices write fewer partials (r x 64 floats per workgroup against
// TM x 64 16-bit values read per run).
struct MColsPlan {
  int S, nsub;
};
static MColsPlan mcols_plan(int64_t M, int64_t C) {
  const int64_t runs = (M + kMColsTM - 1) / kMColsTM;
  const int64_t tiles = (C + kMColsTile - 1) / kMColsTile;
  int64_t S = (1024 + tiles - 1) / tiles;
  if (S > runs) S = runs;
  if (S < 1) S = 1;
  MColsPlan p;
  p.nsub = (int)((runs + S - 1) / S);
  p.S = (int)((runs + p.nsub - 1) / p.nsub);
  return p;
}

// 32-bit offsets within a 256-token run: C < 2^22
static bool cols_use_mfma(int p_dtype, int64_t C) {
  return p_dtype != QL_F32 && C % 8 == 0 && C < ((int64_t)1 << 22);
}

size_t lora_cols_partial_floats(int64_t M, int64_t C, int32_t r) {
  const int64_t s1 = cols_slices(M, C), s2 = mcols_plan(M, C).S;
  return (size_t)(s1 > s2 ? s1 : s2) * (size_t)r * (size_t)C;
}

// The matrix-core form of one product, as a job of a k_cols_mfma launch.
static ColsJob mcols_job(const float *R, int64_t M, const void *P, int64_t C, float scale,
                         bool out_c_major, float *out, float *partial, bool accumulate, int &S) {
  const MColsPlan mp = mcols_plan(M, C);
  S = mp.S;
  // one token slice: the kernel writes the result, no reduction launch
  const ColsOut co{S == 1 ? out : nullptr, scale, out_c_major ? 1 : 0, accumulate ? 1 : 0};
  return ColsJob{R, P, C, partial, co, mp.nsub, (C + kMColsTile - 1) / kMColsTile};
}

// One k_cols_mfma launch over jobs a and b (b.tiles == 0: a alone).
static void launch_mcols(const ColsJob &a, int Sa, const ColsJob &b, int Sb, int64_t M, int32_t r,
                         int p_dtype, const Dropout &dr, bool drop, hipStream_t stream) {
  const int64_t blocks_a = a.tiles * Sa;
  const dim3 grid((unsigned)(blocks_a + b.tiles * Sb));
  const bool rvec = r % 4 == 0;
#define QL_COLS_M(JTV, RV, DRV)                                                               \
  hipLaunchKernelGGL((k_cols_mfma<kMColsTM, JTV, AT, RV, DRV>), grid, dim3(256), 0, stream, a, \
                     b, blocks_a, M, r, dr)
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
}

int launch_lora_cols(const float *R, int64_t M, int32_t r, const void *P, int p_dtype, int64_t C,
                     float scale, bool out_c_major, float *out, float *partial,
                     hipStream_t stream, bool accumulate, const Dropout *drop,
                     ColsReduce *pending) {
  if (pending) pending->S = 0;
  if (C <= 0) return QL_OK;
  int S;
  const Dropout dr = drop ? *drop : Dropout{0u, 0u, 0u};
  if (cols_use_mfma(p_dtype, C)) {
    const ColsJob a = mcols_job(R, M, P, C, scale, out_c_major, out, partial, accumulate, S);
    launch_mcols(a, S, ColsJob{nullptr, nullptr, 0, nullptr, ColsOut{nullptr, 0.0f, 0, 0}, 1, 0}, 0,
                 M, r, p_dtype, dr, drop != nullptr, stream);
    QL_HIP_CHECK_LAUNCH();
    if (S == 1) return QL_OK;
  } else {
    S = cols_slices(M, C);
    const int64_t slice = (M + S - 1) / S;
    const dim3 grid((unsigned)((C + kColsTC - 1) / kColsTC), (unsigned)S);
    with_type(p_dtype, [&](auto *pt) {
      using PT = elem_of<decltype(pt)>;
      if (drop)
        hipLaunchKernelGGL((k_lora_cols<PT, true>), grid, dim3(256), 0, stream, R, M, r, P, C,
                           slice, partial, dr);
      else
        hipLaunchKernelGGL((k_lora_cols<PT, false>), grid, dim3(256), 0, stream, R, M, r, P, C,
                           slice, partial, dr);
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

int launch_lora_cols2(const float *Ra, const void *Pa, int64_t Ca, float scale_a, bool cmaj_a,
                      float *out_a, float *partial_a, const float *Rb, const void *Pb, int64_t Cb,
                      float scale_b, bool cmaj_b, float *out_b, float *partial_b, int64_t M,
                      int32_t r, int p_dtype, hipStream_t stream, bool accumulate,
                      ColsReduce *pending_a, ColsReduce *pending_b) {
  if (!(cols_use_mfma(p_dtype, Ca) && cols_use_mfma(p_dtype, Cb) && Ca > 0 && Cb > 0)) {
    int st = launch_lora_cols(Ra, M, r, Pa, p_dtype, Ca, scale_a, cmaj_a, out_a, partial_a, stream,
                              accumulate, nullptr, pending_a);
    if (st) return st;
    return launch_lora_cols(Rb, M, r, Pb, p_dtype, Cb, scale_b, cmaj_b, out_b, partial_b, stream,
                            accumulate, nullptr, pending_b);
  }
  int Sa, Sb;
  const ColsJob a = mcols_job(Ra, M, Pa, Ca, scale_a, cmaj_a, out_a, partial_a, accumulate, Sa);
  const ColsJob b = mcols_job(Rb, M, Pb, Cb, scale_b, cmaj_b, out_b, partial_b, accumulate, Sb);
  launch_mcols(a, Sa, b, Sb, M, r, p_dtype, Dropout{0u, 0u, 0u}, false, stream);
  QL_HIP_CHECK_LAUNCH();
  *pending_a = Sa == 1 ? ColsReduce{nullptr, 0, 0, 0, 0.0f, 0, 0, nullptr}
                       : ColsReduce{partial_a, Sa, r, Ca, scale_a, cmaj_a ? 1 : 0,
                                    accumulate ? 1 : 0, out_a};
  *pending_b = Sb == 1 ? ColsReduce{nullptr, 0, 0, 0, 0.0f, 0, 0, nullptr}
                       : ColsReduce{partial_b, Sb, r, Cb, scale_b, cmaj_b ? 1 : 0,
                                    accumulate ? 1 : 0, out_b};
  return QL_OK;
}

}  // namespace qlora
