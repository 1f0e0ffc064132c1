// gemv.hip -- decode-sized forward of the QLoRA layer (M <= 16 tokens, 16-bit
// activations: bf16, or fp16 as the compute dtype of Gemma lesson 09, sec.
// 9.3):
//
//   u = x A^T,   y = x W^^T + s u B^T     (26. QLoRA and 4bit Quantization, Step 3)
//
// Memory-bound: the packed 4-bit weight is the dominant traffic, so the
// weight is read exactly once, in as many independent streams as the chip
// can keep in flight, and nothing else competes with it for the load path.
// Two launches:
//
//  k_dec_main   two kinds of workgroups in one grid.  The first compute
//               u = x A^T, one 16-rank tile over one slice of the
//               contraction each (A is read once in total, not once per
//               weight tile), and write fp32 partial sums.  The others stream the weight: a workgroup
//               owns 64 consecutive weight rows and one slice of the
//               contraction; each of its 4 waves owns all 64 rows over a
//               contiguous run of 128-column chunks and reads them straight
//               into matrix-core operand registers (no LDS staging, no
//               barrier until the final cross-wave sum), prefetching the next
//               chunk while it multiplies the current one.  Each workgroup
//               writes its fp32 sums of x W^^T for its slice.
//  k_dec_finish sums the slices in a fixed order and forms
//               y = RN(fmaf(s, sum_j u_j B_nj, base)), and u_save.
//
// Matrix-core op v_mfma_f32_16x16x32_{bf16,f16} (gfx950): A lane l holds
// A[l % 16][8*(l/16) .. +8], B lane l holds B[8*(l/16) .. +8][l % 16], result
// lane l holds D[4*(l/16) .. +4][l % 16].  A = activations (token rows), B =
// 16 weight rows (columns of D).  For one 128-column chunk, lane group q =
// l / 16 loads the 16 packed bytes [16 q, 16 q + 16) of the chunk's 64 bytes
// of its weight row, so a wave load covers 64 contiguous bytes of each of 16
// rows; op j (j = 0..3) takes the 4-byte word j of those 16 bytes, i.e.
// columns 32 q + 8 j + 0..7 of the chunk, and the activation operand of op j
// holds the same columns.
//
// The weight operand is the *unscaled* codebook value of each index (26.
// ..., Step 4 lookup table; a byte -> two 16-bit values table in LDS); the
// block constant is applied to the op's fp32 sums afterwards (26. ..., Step
// 4: table[index] * scale, with the scale taken out of the sum it
// multiplies).  A chunk holds two 64-element blocks per row (lane groups 0-1
// the first, 2-3 the second), and one op sums over all four lane groups, so
// each op runs twice: once with the activation operand of lane groups 2-3
// zeroed (the first block) and once with that of 0-1 zeroed (the second).
// The zeroed operands are built once per chunk and serve all 64 rows.
#include "kernels.h"
#include "upart.h"

namespace qlora {

constexpr int kDecWaves = 4;
constexpr int kDecThreads = 64 * kDecWaves;
constexpr int kDecRows = 64;   // weight rows per workgroup (4 groups of 16, every wave all of them)
constexpr int kDecChunk = 128; // columns per chunk: 64 packed bytes per row

__device__ __forceinline__ float nf4_immediate(int i) {
  constexpr float cb[16] = QL_NF4_CODEBOOK_VALUES;
  float v = cb[0];
#pragma unroll
  for (int k = 1; k < 16; ++k) v = (i == k) ? cb[k] : v;
  return v;
}

// One chunk's loads for one lane: activation operand words (4 ops), the 16
// packed bytes of each of the 4 row groups, and the raw block constants of
// the chunk's two blocks per row group (int8 code + sigma, or fp32 absmax).
struct DecChunk {
  u32x4 xv[4];
  u32x4 wv[4];
  int cq[4][2];
  float cs[4][2];
};

// grid.x = U JT + G S (JT = ceil(r / 16)).  Workgroups [0, U JT): u, rank
// tile b % JT over contraction slice b / JT of uc chunks, partial sums to
// upart [U][M][r].  The rest: row set b / S (64 rows), contraction
// split b % S (cps chunks, waves cpw chunks each), partial sums to part
// [S][M][N].
template <typename AT, typename LT, bool DQ, bool EV, bool VC>
__global__ __launch_bounds__(kDecThreads, 3) void k_dec_main(
    const uint16_t *__restrict__ x, int M, const uint8_t *__restrict__ packed, BlockScales sc,
    int64_t N, int64_t K, const LT *__restrict__ A, int32_t r, float *__restrict__ part,
    float *__restrict__ upart, int S, int U, int cpw, int uc, Dropout dr) {
  __shared__ uint32_t lut[256];
  __shared__ float red[kDecWaves][16][kDecRows];
  const int t = threadIdx.x;
  const int wave = t >> 6, lane = t & 63;
  const int nl = lane & 15, q = lane >> 4;
  const int64_t NC = (K + kDecChunk - 1) / kDecChunk;
  // token row of this lane's activation operand (rows past M repeat the
  // last one; their results are never stored)
  const int m = nl < M ? nl : M - 1;

  const int JT = (r + 15) / 16;
  if ((int)blockIdx.x < U * JT) {
    u_slice_tile<AT, LT>(x, M, K, A, r, upart, uc, blockIdx.x / JT, blockIdx.x % JT, 0,
                         &red[0][0][0], dr);
    return;
  }

  // ---------------- x W^^T over this workgroup's rows and slice --------------
  if (t < 256) {
    const uint16_t lo = Half<AT>::bits(nf4_immediate(t >> 4));
    const uint16_t hi = Half<AT>::bits(nf4_immediate(t & 15));
    lut[t] = (uint32_t)lo | ((uint32_t)hi << 16);  // element 2i (high nibble) first
  }
  const int64_t b = (int64_t)blockIdx.x - (int64_t)U * JT;
  const int64_t row0 = (b / S) * kDecRows;
  const int sp = (int)(b % S);
  const int64_t cps = VC ? (int64_t)kDecWaves * cpw : (NC + S - 1) / S;
  const int64_t s_end = (sp + 1) * cps < NC ? (sp + 1) * cps : NC;
  const int64_t c_begin = sp * cps + (int64_t)wave * cpw;
  const int64_t c_end = c_begin + cpw < s_end ? c_begin + cpw : s_end;
  const int nloc = c_end > c_begin ? (int)(c_end - c_begin) : 0;

  const int64_t KB = K >> 6;
  const int64_t row_bytes = K >> 1;
  const uint8_t *wsrc[4];
  int64_t srow[4];
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const int64_t n = row0 + 16 * g + nl < N ? row0 + 16 * g + nl : N - 1;
    wsrc[g] = packed + n * row_bytes;
    srow[g] = n * KB;
  }
  const uint16_t *xsrc = x + (int64_t)m * K;
  const float mu = DQ ? sc.mu[0] : 0.0f;
  const bool lo_lane = q < 2;
  // VC: the codes of all of this wave's chunks (2 cpw <= 16 bytes per row,
  // starting at a multiple of 2 cpw) as one aligned 16-byte load per row
  // group, and their one sigma (the 2 cpw blocks lie in one group of 256)
  u32x4 cvec[4];
  float cvs[4];
  int cvo[4];
  if constexpr (VC) {
    const int64_t cb = c_begin < NC ? c_begin : NC - 1;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int64_t i0 = srow[g] + 2 * cb;
      cvo[g] = (int)(i0 & 15);
      cvec[g] = *reinterpret_cast<const u32x4 *>(sc.q + (i0 & ~(int64_t)15));
      cvs[g] = sc.sigma[i0 >> 8];
    }
  }
  // Every load is unconditional, at an index clamped into the array (the
  // last chunk of a contraction with K % 128 == 64 has only its first block:
  // lane groups 2-3 re-read the first half and that block's constant is 0).
  auto load_chunk = [&](int64_t c, DecChunk &R) {
    const int64_t col = c * kDecChunk;
    const bool two = EV || col + 64 < K;
    const int qe = (two || q < 2) ? q : q - 2;
    const uint16_t *xp = xsrc + col + 32 * qe;
#pragma unroll
    for (int j = 0; j < 4; ++j) R.xv[j] = *reinterpret_cast<const u32x4 *>(xp + 8 * j);
#pragma unroll
    for (int g = 0; g < 4; ++g)
      R.wv[g] = *reinterpret_cast<const u32x4 *>(wsrc[g] + 64 * c + 16 * qe);
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      if constexpr (VC) {
      } else if constexpr (EV) {
        // blocks of 64 and K % 128 == 0: the chunk's two block constants
        // start at an even index and share one sigma; the two codes as one
        // 2-byte load
        const int64_t bi = srow[g] + 2 * c;
        if constexpr (DQ) {
          R.cq[g][0] = (int)*reinterpret_cast<const uint16_t *>(sc.q + bi);
          R.cs[g][0] = sc.sigma[bi >> 8];
        } else {
          const float2 a = *reinterpret_cast<const float2 *>(sc.absmax + bi);
          R.cs[g][0] = a.x;
          R.cs[g][1] = a.y;
        }
      } else {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int64_t bi = sc.index(srow[g] + 2 * c + (two ? h : 0));
          if constexpr (DQ) {
            R.cq[g][h] = sc.q[bi];
            R.cs[g][h] = sc.sigma[bi >> 8];
          } else {
            R.cq[g][h] = 0;
            R.cs[g][h] = sc.absmax[bi];
          }
        }
      }
    }
  };
  // the chunk's two block constants of row group g
  auto consts = [&](const DecChunk &R, int64_t c, int g, bool two, float &a0, float &a1) {
    if constexpr (VC) {
      const int o = cvo[g] + 2 * (int)(c - c_begin);
      const uint32_t d = cvec[g][o >> 2] >> (8 * (o & 3));
      a0 = __builtin_fmaf((float)(int8_t)(d & 0xFF), cvs[g], mu);
      a1 = __builtin_fmaf((float)(int8_t)((d >> 8) & 0xFF), cvs[g], mu);
    } else if constexpr (EV) {
      if constexpr (DQ) {
        a0 = __builtin_fmaf((float)(int8_t)(R.cq[g][0] & 0xFF), R.cs[g][0], mu);
        a1 = __builtin_fmaf((float)(int8_t)(R.cq[g][0] >> 8), R.cs[g][0], mu);
      } else {
        a0 = R.cs[g][0];
        a1 = R.cs[g][1];
      }
    } else {
      a0 = DQ ? __builtin_fmaf((float)R.cq[g][0], R.cs[g][0], mu) : R.cs[g][0];
      const float a1h = DQ ? __builtin_fmaf((float)R.cq[g][1], R.cs[g][1], mu) : R.cs[g][1];
      a1 = two ? a1h : 0.0f;
    }
  };

  f32x4 yacc[4];
#pragma unroll
  for (int g = 0; g < 4; ++g) yacc[g] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](const DecChunk &R, int64_t c) {
    const bool two = EV || c * kDecChunk + 64 < K;
    u32x4 xl[4], xh[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        xl[j][d] = lo_lane ? R.xv[j][d] : 0u;
        xh[j][d] = lo_lane ? 0u : R.xv[j][d];
      }
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      float a0, a1;
      consts(R, c, g, two, a0, a1);
      f32x4 pl = {0.f, 0.f, 0.f, 0.f}, ph = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t w = R.wv[g][j];
        const u32x4 wo = {lut[w & 0xFF], lut[(w >> 8) & 0xFF], lut[(w >> 16) & 0xFF], lut[w >> 24]};
        pl = Half<AT>::mfma16(xl[j], wo, pl);
        ph = Half<AT>::mfma16(xh[j], wo, ph);
      }
      // pl[v] / ph[v]: sum over the chunk's first / second block of
      // x[4q + v][k] * cb[idx[n][k]], n = row0 + 16 g + nl
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        yacc[g][v] = __builtin_fmaf(a0, pl[v], yacc[g][v]);
        yacc[g][v] = __builtin_fmaf(a1, ph[v], yacc[g][v]);
      }
    }
  };

  DecChunk R0, R1;
  if (nloc > 0) load_chunk(c_begin, R0);
  __syncthreads();  // lut
  if (nloc == 1) {
    compute(R0, c_begin);
  } else if (nloc > 1) {
    // two register sets: the loads of chunk i + 1 fly while chunk i is
    // multiplied (the last iteration re-reads the last chunk, from cache)
    for (int i = 0; i < nloc; i += 2) {
      load_chunk(c_begin + (i + 1 < nloc ? i + 1 : nloc - 1), R1);
      compute(R0, c_begin + i);
      if (i + 1 >= nloc) break;
      load_chunk(c_begin + (i + 2 < nloc ? i + 2 : nloc - 1), R0);
      compute(R1, c_begin + i + 1);
    }
  }

  // yacc[g][v] = partial y[4q + v][row0 + 16 g + nl]: sum over the waves
#pragma unroll
  for (int g = 0; g < 4; ++g)
#pragma unroll
    for (int v = 0; v < 4; ++v) red[wave][4 * q + v][16 * g + nl] = yacc[g][v];
  __syncthreads();
  for (int e = t; e < M * kDecRows; e += kDecThreads) {
    const int mo = e / kDecRows, n = e % kDecRows;
    float sum = 0.0f;
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) sum += red[w][mo][n];
    if (row0 + n < N) part[((int64_t)sp * M + mo) * N + row0 + n] = sum;
  }
}

// y[m][n] = RN(fmaf(s, sum_j u[m][j] B[n][j], sum over splits of x W^^T)),
// u[m][j] = uscale * (sum over the u slices in order) (both sums start from
// 0 and add in slice order; the rank sum is a chain of fmaf in rank order;
// uscale is 1, or 1 / (1 - p) under LoRA dropout).  Grid
// (ceil(N / 256), M): one thread per output; the workgroups of the first
// column store u_save.  Slices are read 8 at a time with all 8 loads in
// flight (at clamped indices), so S slices cost ceil(S / 8) round trips.
template <typename AT, typename LT>
__global__ __launch_bounds__(256) void k_dec_finish(const float *__restrict__ part, int S,
                                                    const float *__restrict__ upart, int U, int M,
                                                    int64_t N, int32_t r,
                                                    const LT *__restrict__ B, float s,
                                                    uint16_t *__restrict__ y,
                                                    float *__restrict__ u_save, float uscale) {
  __shared__ float us[128];
  const int t = threadIdx.x;
  const int mo = blockIdx.y;
  const int64_t n = (int64_t)blockIdx.x * 256 + t;
  const int64_t nc = n < N ? n : N - 1;
  // the first 8 slice partials of y, the first 8 of u (threads t < r) and
  // the row of B (at most 128 values: 16 pieces of 8) are all issued before
  // the first sum
  const int tj = t < r ? t : r - 1;
  float pv[8], uv[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int ii = i < S ? i : S - 1;
    pv[i] = part[((int64_t)ii * M + mo) * N + nc];
  }
  if (t < r) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int iu = i < U ? i : U - 1;
      uv[i] = upart[((int64_t)iu * M + mo) * r + tj];
    }
  }
  const LT *bp = B + nc * r;
  u32x4 bw[16 * sizeof(LT) / 2];
  const int np = r % 8 == 0 ? r / 8 : 0;
#pragma unroll
  for (int i = 0; i < 16; ++i)
    if (i < np) {
      if constexpr (sizeof(LT) == 2) {
        bw[i] = *reinterpret_cast<const u32x4 *>(bp + 8 * i);
      } else {
        bw[2 * i] = *reinterpret_cast<const u32x4 *>(bp + 8 * i);
        bw[2 * i + 1] = *reinterpret_cast<const u32x4 *>(bp + 8 * i + 4);
      }
    }
  float base = 0.0f, su = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i)
    if (i < S) base += pv[i];
  for (int i0 = 8; i0 < S; i0 += 8) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int ii = i0 + i < S ? i0 + i : S - 1;
      pv[i] = part[((int64_t)ii * M + mo) * N + nc];
    }
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (i0 + i < S) base += pv[i];
  }
  if (t < r) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (i < U) su += uv[i];
    for (int i0 = 8; i0 < U; i0 += 8) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int iu = i0 + i < U ? i0 + i : U - 1;
        uv[i] = upart[((int64_t)iu * M + mo) * r + tj];
      }
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (i0 + i < U) su += uv[i];
    }
    su = uscale * su;
    us[t] = su;
    if (u_save && blockIdx.x == 0) u_save[(int64_t)mo * r + t] = su;
  }
  __syncthreads();
  if (n >= N) return;
  float l = 0.0f;
  if (np > 0) {
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (i < np) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          float bv;
          if constexpr (sizeof(LT) == 2)
            bv = (e & 1) ? Half<LT>::hi(bw[i][e >> 1]) : Half<LT>::lo(bw[i][e >> 1]);
          else
            bv = __uint_as_float(bw[2 * i + (e >> 2)][e & 3]);
          l = __builtin_fmaf(us[8 * i + e], bv, l);
        }
      }
  } else {
    for (int j = 0; j < r; ++j) l = __builtin_fmaf(us[j], load_as_f32(B, n * r + j), l);
  }
  y[(int64_t)mo * N + n] = Half<AT>::bits(__builtin_fmaf(s, l, base));
}

int launch_fwd_finish(int act_dtype, int lora_dtype, const float *part, int S,
                      const float *upart, int U, int64_t M, int64_t N, int32_t r, const void *B,
                      float s, void *y, float *u_save, hipStream_t stream, float uscale) {
  const dim3 fgrid((unsigned)((N + 255) / 256), (unsigned)M);
  with_half(act_dtype, [&](auto *tag) {
    using AT = elem_of<decltype(tag)>;
    if (lora_dtype == QL_F32)
      hipLaunchKernelGGL((k_dec_finish<AT, float>), fgrid, dim3(256), 0, stream, part, S, upart,
                         U, (int)M, N, r, (const float *)B, s, (uint16_t *)y, u_save, uscale);
    else
      hipLaunchKernelGGL((k_dec_finish<AT, AT>), fgrid, dim3(256), 0, stream, part, S, upart, U,
                         (int)M, N, r, (const AT *)B, s, (uint16_t *)y, u_save, uscale);
  });
  QL_HIP_CHECK_LAUNCH();
  return QL_OK;
}

// Launch plan of a decode forward.
struct DecPlan {
  int S;     // contraction splits of the weight stream
  int cpw;   // chunks per wave
  int U;     // u slices
  int uc;    // chunks per u slice
  int64_t G; // row sets of 64
  bool ev;   // blocks of 64 and K % 128 == 0: two block constants per chunk, one sigma
  bool vc;   // ... with double quantisation and runs of cpw = 2^k <= 8 chunks whose
             // codes sit at a multiple of 2 cpw: one code load per wave and row group
};

// The weight stream is cut into wave-tasks of cpw consecutive 128-column
// chunks of 64 rows; a workgroup's 4 waves cover 4 cpw consecutive chunks,
// so the contraction is split in S slices.  The kernel's register use
// allows 3 resident workgroups of 4 waves per compute unit (256 units).
// With double quantisation and K % 128 == 0, cpw is the largest power of
// two up to 8 that still gives at least half of the resident workgroups (1.5
// per unit: measured over cpw = 1..8 on weights from 4096x4096 to
// 8192x28672, longer runs per wave beat a second, partial round of
// workgroups) and keeps each wave's 2 cpw codes inside one aligned 16-byte
// piece (K / 64 a multiple of 2 cpw, N K / 64 of 16), so a wave loads the
// block constants of all its chunks at once.  Otherwise cpw stays 1 while the tasks fill the resident
// workgroups; beyond that each wave takes several consecutive chunks.  In
// both, a wave's loads of its next chunk are in flight while it multiplies
// the current one.  u takes one workgroup per 4 chunks, at most 16.
static DecPlan dec_plan(int64_t N, int64_t K, bool dq, int shift) {
  DecPlan p;
  const int64_t NC = (K + kDecChunk - 1) / kDecChunk;
  const int64_t KB = K >> 6;
  p.G = (N + kDecRows - 1) / kDecRows;
  p.ev = K % 128 == 0 && shift == 0;
  p.vc = false;
  const int64_t resident = (int64_t)256 * 3;
  if (p.ev && dq && (N * KB) % 16 == 0) {
    int c = 8;
    while (c > 1 && (KB % (2 * c) != 0 ||
                     p.G * ((NC + kDecWaves * c - 1) / (kDecWaves * c)) < resident / 2))
      c >>= 1;
    if (KB % (2 * c) == 0) {
      p.vc = true;
      p.cpw = c;
      p.S = (int)((NC + kDecWaves * c - 1) / (kDecWaves * c));
    }
  }
  if (!p.vc) {
    const int64_t tasks = p.G * NC, cap = resident * kDecWaves;
    p.cpw = (int)(tasks <= cap ? 1 : (tasks + cap - 1) / cap);
    int64_t S = (NC + (int64_t)kDecWaves * p.cpw - 1) / ((int64_t)kDecWaves * p.cpw);
    const int64_t cps = (NC + S - 1) / S;
    p.S = (int)((NC + cps - 1) / cps);
  }
  const USlices us = u_slices(K);
  p.U = us.U;
  p.uc = us.uc;
  return p;
}

size_t gemv_fwd_partial_floats(int64_t M, int64_t N, int64_t K, int32_t r) {
  // the largest of the plans of the weight's formats
  const DecPlan p = dec_plan(N, K, false, 0), p2 = dec_plan(N, K, true, 0);
  if (p2.S > p.S) return (size_t)p2.S * M * N + (size_t)p2.U * M * r;
  return (size_t)p.S * M * N + (size_t)p.U * M * r;
}

// A 16-bit LoRA factor has the activations' format (checked by the caller).
// part: gemv_fwd_partial_floats floats of workspace.
int launch_gemv_fwd(const void *xv, int act_dtype, int64_t M, const uint8_t *packed,
                    BlockScales sc, int64_t N, int64_t K, const void *A, const void *B,
                    int lora_dtype, int32_t r, float s, void *yv, float *u_save,
                    hipStream_t stream, float *part, const Dropout *drop, float dscale) {
  const Dropout dr = drop ? *drop : Dropout{0u, 0u, 0u};
  const uint16_t *x = (const uint16_t *)xv;
  uint16_t *y = (uint16_t *)yv;
  const bool dq = sc.absmax == nullptr;
  const DecPlan p = dec_plan(N, K, dq, sc.shift);
  float *upart = part + (size_t)p.S * M * N;
  const dim3 grid((unsigned)(p.U * ((r + 15) / 16) + p.G * p.S));
  with_half(act_dtype, [&](auto *tag) {
    using AT = elem_of<decltype(tag)>;
    auto go = [&](auto *ltag) {
      using LT = elem_of<decltype(ltag)>;
      auto main = [&](auto dqt, auto evt, auto vct) {
        hipLaunchKernelGGL((k_dec_main<AT, LT, decltype(dqt)::value, decltype(evt)::value,
                                       decltype(vct)::value>),
                           grid, dim3(kDecThreads), 0, stream, x, (int)M, packed, sc, N, K,
                           (const LT *)A, r, part, upart, p.S, p.U, p.cpw, p.uc, dr);
      };
      using T = std::true_type;
      using F = std::false_type;
      if (p.vc) main(T{}, T{}, T{});
      else if (dq && p.ev) main(T{}, T{}, F{});
      else if (dq) main(T{}, F{}, F{});
      else if (p.ev) main(F{}, T{}, F{});
      else main(F{}, F{}, F{});

    };
    if (lora_dtype == QL_F32) go((float *)nullptr);
    else go((AT *)nullptr);
  });
  QL_HIP_CHECK_LAUNCH();
  return launch_fwd_finish(act_dtype, lora_dtype, part, p.S, upart, p.U, M, N, r, B, s, y, u_save,
                           stream, drop ? dscale : 1.0f);
}

}  // namespace qlora
