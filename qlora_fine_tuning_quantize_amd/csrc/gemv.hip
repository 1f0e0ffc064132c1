// gemv.hip -- decode-sized forward of the QLoRA layer (M <= 16 tokens, 16-bit
// activations: bf16, or fp16 as the compute dtype of Gemma lesson 09, sec.
// 9.3), one kernel launch per call (two when the contraction is split, below):
//
//   u = x A^T,   y = x W^^T + s u B^T     (26. QLoRA and 4bit Quantization, Step 3)
//
// Memory-bound: the packed 4-bit weight is the dominant traffic.  Each
// workgroup owns 16 consecutive weight rows, which are one contiguous span of
// the packed array.  The contraction runs in rounds of 64 NF4 blocks (4096
// columns): the round's slice of the 16 rows is read with 16-byte loads, each
// wave instruction covering half a kilobyte of two rows, and staged in LDS;
// the 8 waves then split the round's blocks and read their codes back in the
// matrix-core operand layout.  The round's block constants (absmax, or the
// double-quantised form q * sigma + mu) are resolved once into an LDS table.
//
// The 16x16x32 16-bit matrix-core op multiplies the activations by the
// *unscaled* codebook values of one 64-element chunk (16 rows x 32 columns
// per op, two ops per chunk; a chunk lies inside one NF4 block of 64 or 128);
// the block's fp32 constant is then applied to the 4 partial sums each lane
// holds (26. ..., Step 4: table[index] * scale, with the scale taken out of
// the 64-term sum it multiplies).  The codebook lookup
// goes through a byte -> 2 x 16-bit table in LDS built from immediates.
//
// The rank-r pre-product u = x A^T is recomputed by every workgroup from the
// activation operand it already holds (extra 16x16x32 ops against rows of A,
// read from L2), so decode needs no u kernel and no grid-wide dependency.
// Workgroup 0 stores u when the caller asks for it.
//
// A weight with few row groups and a long contraction would leave most
// compute units idle; there grid.y splits the contraction into whole rounds,
// each split writes its fp32 sums of y and u to the caller's workspace, and
// k_gemv_reduce adds the splits in order and forms y as the single-split
// epilogue does.
//
// Operand layout of v_mfma_f32_16x16x32_{bf16,f16} (gfx950): A lane l holds
// A[l % 16][8*(l/16) .. +8], B lane l holds B[8*(l/16) .. +8][l % 16], and the
// result lane l holds D[4*(l/16) .. +4][l % 16].  All operands use the same
// permutation of K within a block: op c of block b covers
// k = 64 b + 16 q + 8 c + e for lane group q = l / 16 and e = 0..7.
#include "kernels.h"

namespace qlora {

constexpr int kGemvRows = 16;
constexpr int kGemvWaves = 8;
constexpr int kGemvThreads = 64 * kGemvWaves;
constexpr int kGemvRound = 64;  // NF4 blocks per row per round
// LDS stride of one staged row: 16 bytes of padding put the 8-byte reads of
// 16 rows x 4 lane groups at the same column offset on distinct banks.
constexpr int kGemvRowStride = kGemvRound * 32 + 16;
// 16-byte weight chunks per lane per round (16 rows x 2 KB / 512 lanes)
constexpr int kGemvChunks = kGemvRows * kGemvRound * 2 / kGemvThreads;
// NF4 block constants per lane per round
constexpr int kGemvScales = kGemvRows * kGemvRound / kGemvThreads;
// LDS stride of one staged activation row (a round of 16-bit values + 16 bytes)
constexpr int kGemvXStride = kGemvRound * 128 + 16;

// Blocks whose activation and A loads are in flight together: 8 for a
// 16-wide rank tile in 16 bits at 2 waves per SIMD, fewer as the per-block
// register footprint grows or as more waves share the registers.
template <typename LT, int JT, int WPE>
constexpr int gemv_batch() {
  constexpr int w = JT * (int)(sizeof(LT) / 2) * (WPE / 2);
  return w >= 8 ? 1 : 8 / w;
}

__device__ __forceinline__ float nf4_immediate(int i) {
  constexpr float cb[16] = QL_NF4_CODEBOOK_VALUES;
  float v = cb[0];
#pragma unroll
  for (int k = 1; k < 16; ++k) v = (i == k) ? cb[k] : v;
  return v;
}

// 16 consecutive LoRA-A values of one rank row, kept raw until use; half(c)
// gives values 8c .. 8c + 7 as a matrix-core operand in format AT.  LT is
// AT (used as loaded) or float.
template <typename AT, typename LT>
struct ARaw {
  u32x4 v[2];
  __device__ __forceinline__ void load(const LT *p) {
    v[0] = reinterpret_cast<const u32x4 *>(p)[0];
    v[1] = reinterpret_cast<const u32x4 *>(p)[1];
  }
  __device__ __forceinline__ u32x4 half(int c) const { return v[c]; }
};
template <typename AT>
struct ARaw<AT, float> {
  float4 v[4];
  __device__ __forceinline__ void load(const float *p) {
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = reinterpret_cast<const float4 *>(p)[i];
  }
  __device__ __forceinline__ u32x4 half(int c) const {
    const float4 a = v[2 * c], b = v[2 * c + 1];
    return u32x4{Half<AT>::pack2(a.x, a.y), Half<AT>::pack2(a.z, a.w), Half<AT>::pack2(b.x, b.y),
                 Half<AT>::pack2(b.z, b.w)};
  }
};

// Per-block register operands of one lane: 2 x 8 activations and JT x 16 A values.
template <typename AT, typename LT, int JT>
struct GemvBlock {
  u32x4 x0, x1;
  ARaw<AT, LT> a[JT];
};

// XM > 0: the round's activations of all M <= XM token rows are staged in
// LDS once per workgroup (the operand layout repeats a token row across the
// 16 lanes of a lane group, which would otherwise be 16 / M copies of the
// same bytes through the load path); XM = 0: read in operand layout.
// WPE: waves per SIMD the register allocation must allow.  2 (one workgroup
// per compute unit) leaves the most registers for loads in flight, which is
// what a grid of at most one workgroup per unit needs; 4 lets two workgroups
// share a unit, so that a larger grid overlaps one workgroup's round trips
// with the other's work.
template <typename AT, typename LT, int JT, bool DQ, int XM, int WPE>
__global__ __launch_bounds__(kGemvThreads, WPE) void k_gemv_fwd(const uint16_t *__restrict__ x, int M,
                                                           const uint8_t *__restrict__ packed,
                                                           BlockScales sc, int64_t N, int64_t K,
                                                           const LT *__restrict__ A,
                                                           const LT *__restrict__ B, int32_t r,
                                                           float s, uint16_t *__restrict__ y,
                                                           float *__restrict__ u_save,
                                                           float *__restrict__ part) {
  __shared__ uint32_t lut[256];
  __shared__ __attribute__((aligned(16))) uint8_t wt[kGemvRows * kGemvRowStride];
  __shared__ __attribute__((aligned(16))) uint8_t xs[XM > 0 ? XM * kGemvXStride : 16];
  __shared__ float scl[kGemvRows][kGemvRound];
  __shared__ float red[kGemvWaves][16][16];
  __shared__ float ured[kGemvWaves][16][16 * JT];
  __shared__ float us[16][16 * JT];
  __shared__ float bs[16][16 * JT];
  const int t = threadIdx.x;
  const int wave = t >> 6, lane = t & 63;
  const int nl = lane & 15, q = lane >> 4;
  const int64_t n0 = (int64_t)blockIdx.x * kGemvRows;
  // Token rows past M and rank rows past r are clamped to valid ones: they
  // only produce outputs that are never stored or summed.
  const int m = nl < M ? nl : M - 1;
  const int64_t KB = K >> 6;
  const int64_t row_bytes = K >> 1;
  const uint16_t *xrow = x + (int64_t)m * K + 16 * q;
  const LT *arow[JT];
#pragma unroll
  for (int jt = 0; jt < JT; ++jt) {
    const int j = 16 * jt + nl < r ? 16 * jt + nl : r - 1;
    arow[jt] = A + (int64_t)j * K + 16 * q;
  }
  const float mu = DQ ? sc.mu[0] : 0.0f;

  // Every load below is unconditional, its index clamped into the array:
  // a load under a branch makes the compiler wait for it at the join, which
  // would serialise the round trips this kernel overlaps.  Values loaded for
  // clamped indices are masked where they are stored.
  // This workgroup's rows of B: loaded first, staged in LDS with the first round.
  constexpr int kBPer = (16 * 16 * JT + kGemvThreads - 1) / kGemvThreads;
  float bv[kBPer];
#pragma unroll
  for (int i = 0; i < kBPer; ++i) {
    const int e = t + kGemvThreads * i;
    const int row = (e / (16 * JT)) & 15, j = e % (16 * JT);
    const int64_t nn = n0 + row < N ? n0 + row : N - 1;
    bv[i] = load_as_f32(B, nn * r + (j < r ? j : r - 1));
  }
  if (t < 256) {
    const uint16_t hi = Half<AT>::bits(nf4_immediate(t >> 4));
    const uint16_t lo = Half<AT>::bits(nf4_immediate(t & 15));
    lut[t] = (uint32_t)hi | ((uint32_t)lo << 16);
  }

  constexpr int kBatch = gemv_batch<LT, JT, WPE>();
  constexpr int kWaveBlocks = kGemvRound / kGemvWaves;  // blocks per wave per full round
  GemvBlock<AT, LT, JT> bl[kBatch];
  // loads of blocks first .. first + kBatch - 1 of the round, clamped to its last block
  auto load_batch = [&](int64_t rb0, int first, int RB) {
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const int64_t b = rb0 + (first + i < RB ? first + i : RB - 1);
      if constexpr (XM == 0) {
        const u32x4 *xp = reinterpret_cast<const u32x4 *>(xrow + 64 * b);
        bl[i].x0 = xp[0];
        bl[i].x1 = xp[1];
      }
#pragma unroll
      for (int jt = 0; jt < JT; ++jt) bl[i].a[jt].load(arow[jt] + 64 * b);
    }
  };

  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  f32x4 uacc[JT], uacc1[1];
  uacc1[0] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int jt = 0; jt < JT; ++jt) uacc[jt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // contraction split blockIdx.y of gridDim.y: whole rounds rb_begin .. rb_end
  const int64_t rounds = (KB + kGemvRound - 1) / kGemvRound;
  const int64_t per = (rounds + gridDim.y - 1) / gridDim.y;
  const int64_t rb_begin = (int64_t)blockIdx.y * per * kGemvRound;
  const int64_t rb_end = rb_begin + per * kGemvRound < KB ? rb_begin + per * kGemvRound : KB;
  for (int64_t rb0 = rb_begin; rb0 < rb_end; rb0 += kGemvRound) {
    const int RB = KB - rb0 < kGemvRound ? (int)(KB - rb0) : kGemvRound;
    // the round's weight slice: 16 rows x 2 RB chunks of 16 bytes; chunk c is
    // column chunk c % 128 of row c / 128 (chunks past the slice or rows past
    // N re-read the slice's first chunk and are not stored)
    u32x4 wv[kGemvChunks];
#pragma unroll
    for (int i = 0; i < kGemvChunks; ++i) {
      const int c = t + kGemvThreads * i;
      const int row = c >> 7, cr = c & 127;
      const bool ok = cr < 2 * RB && n0 + row < N;
      wv[i] = *reinterpret_cast<const u32x4 *>(packed + (n0 + (ok ? row : 0)) * row_bytes +
                                                32 * rb0 + 16 * (ok ? cr : 0));
    }
    // the round's block constants: entry e is block e % 64 of row e / 64
    // (rows past N read the last row), loaded raw and combined only after
    // every load of the round is out
    int qv[kGemvScales];
    float sv[kGemvScales];
#pragma unroll
    for (int i = 0; i < kGemvScales; ++i) {
      const int e = t + kGemvThreads * i;
      const int row = e >> 6, b = e & 63;
      const int64_t nn = n0 + row < N ? n0 + row : N - 1;
      const int64_t g = sc.index(nn * KB + rb0 + (b < RB ? b : RB - 1));
      qv[i] = DQ ? (int)sc.q[g] : 0;
      sv[i] = DQ ? sc.sigma[g >> 8] : sc.absmax[g];
    }
    // the round's activations (XM > 0): row c >> 9, 16-byte chunk c & 511
    u32x4 xv[XM > 0 ? XM : 1];
#pragma unroll
    for (int i = 0; i < XM; ++i) {
      const int c = t + kGemvThreads * i;
      const int row = (c >> 9) < M ? (c >> 9) : M - 1;
      const int cc = (c & 511) < 8 * RB ? (c & 511) : 8 * RB - 1;
      xv[i] = *reinterpret_cast<const u32x4 *>(x + (int64_t)row * K + 64 * rb0 + 8 * cc);
    }
    // this wave's blocks of the round: wb0 .. wb0 + cnt - 1
    const int wb0 = wave * kWaveBlocks;
    const int cnt = RB - wb0 < 0 ? 0 : (RB - wb0 < kWaveBlocks ? RB - wb0 : kWaveBlocks);
    // the first batch's loads go out before the staging stores wait for the
    // weight slice (at rank tile 8 after them: the registers are needed)
    // A full round with activations in LDS and one load batch (one 16-rank
    // tile in 16 bits) issues its A loads only after the staging barrier and
    // runs all weight ops first: the staging stores then wait for the
    // weight slice alone, and the A loads fly during the weight ops.
    const bool late_a = XM > 0 && kBatch == kWaveBlocks && JT < 8 && cnt == kWaveBlocks;
    if constexpr (JT < 8)
      if (!late_a) load_batch(rb0, wb0, RB);
#pragma unroll
    for (int i = 0; i < kGemvChunks; ++i) {
      const int c = t + kGemvThreads * i;
      if ((c & 127) < 2 * RB)
        *reinterpret_cast<u32x4 *>(wt + (c >> 7) * kGemvRowStride + 16 * (c & 127)) = wv[i];
    }
#pragma unroll
    for (int i = 0; i < kGemvScales; ++i) {
      const int e = t + kGemvThreads * i;
      scl[e >> 6][e & 63] = DQ ? __builtin_fmaf((float)qv[i], sv[i], mu) : sv[i];
    }
#pragma unroll
    for (int i = 0; i < XM; ++i) {
      const int c = t + kGemvThreads * i;
      if ((c & 511) < 8 * RB)
        *reinterpret_cast<u32x4 *>(xs + (c >> 9) * kGemvXStride + 16 * (c & 511)) = xv[i];
    }
    if (rb0 == rb_begin) {
#pragma unroll
      for (int i = 0; i < kBPer; ++i) {
        const int e = t + kGemvThreads * i;
        if (e < 16 * 16 * JT)
          bs[e / (16 * JT)][e % (16 * JT)] = (e % (16 * JT)) < r ? bv[i] : 0.0f;
      }
    }
    if constexpr (JT >= 8) load_batch(rb0, wb0, RB);
    __syncthreads();

    // one block, weight part: 2 ops against the unscaled codes, then the
    // block constant; returns the activation operand in xr0, xr1
    auto wpart = [&](const GemvBlock<AT, LT, JT> &g, int bb, u32x4 &xr0, u32x4 &xr1) {
      const u32x2 w =
          *reinterpret_cast<const u32x2 *>(wt + nl * kGemvRowStride + 32 * bb + 8 * q);
      u32x4 wb0v, wb1v;
      wb0v.x = lut[w.x & 0xFF];
      wb0v.y = lut[(w.x >> 8) & 0xFF];
      wb0v.z = lut[(w.x >> 16) & 0xFF];
      wb0v.w = lut[w.x >> 24];
      wb1v.x = lut[w.y & 0xFF];
      wb1v.y = lut[(w.y >> 8) & 0xFF];
      wb1v.z = lut[(w.y >> 16) & 0xFF];
      wb1v.w = lut[w.y >> 24];
      if constexpr (XM > 0) {
        const uint8_t *xp = xs + (m < XM ? m : XM - 1) * kGemvXStride + 128 * bb + 32 * q;
        xr0 = *reinterpret_cast<const u32x4 *>(xp);
        xr1 = *reinterpret_cast<const u32x4 *>(xp + 16);
      } else {
        xr0 = g.x0;
        xr1 = g.x1;
      }
      f32x4 part = {0.f, 0.f, 0.f, 0.f};
      part = Half<AT>::mfma16(xr0, wb0v, part);
      part = Half<AT>::mfma16(xr1, wb1v, part);
      // part[v] = sum over the block of x[4q+v][k] * cb[idx[n][k]] for column n = n0 + nl
      const float a = scl[nl][bb];
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[v] = __builtin_fmaf(a, part[v], acc[v]);
    };
    // one block, bypass part: 2 JT ops against A (at one rank tile, two
    // accumulator chains)
    auto upart = [&](const GemvBlock<AT, LT, JT> &g, const u32x4 &xr0, const u32x4 &xr1) {
#pragma unroll
      for (int jt = 0; jt < JT; ++jt) {
        uacc[jt] = Half<AT>::mfma16(xr0, g.a[jt].half(0), uacc[jt]);
        f32x4 &u1 = JT == 1 ? uacc1[jt] : uacc[jt];
        u1 = Half<AT>::mfma16(xr1, g.a[jt].half(1), u1);
      }
    };
    auto block = [&](const GemvBlock<AT, LT, JT> &g, int bb) {
      u32x4 xr0, xr1;
      wpart(g, bb, xr0, xr1);
      upart(g, xr0, xr1);
    };
    // A wave with all its blocks present (every full round of 4096 columns)
    // runs branch-free, so that the compiler overlaps the LDS reads and the
    // matrix ops of different blocks.
    const bool full = JT < 8 && cnt == kWaveBlocks;  // (rank tile 8: registers are short)
    if (late_a) {
      load_batch(rb0, wb0, RB);
      u32x4 xk0[kWaveBlocks], xk1[kWaveBlocks];
#pragma unroll
      for (int i = 0; i < kWaveBlocks; ++i) wpart(bl[i], wb0 + i, xk0[i], xk1[i]);
#pragma unroll
      for (int i = 0; i < kWaveBlocks; ++i) upart(bl[i], xk0[i], xk1[i]);
    } else {
#pragma unroll
      for (int i0 = 0; i0 < kWaveBlocks; i0 += kBatch) {
        if (i0 > 0) load_batch(rb0, wb0 + i0, RB);
        if (full) {
#pragma unroll
          for (int i = 0; i < kBatch; ++i) block(bl[i], wb0 + i0 + i);
        } else {
#pragma unroll
          for (int i = 0; i < kBatch; ++i)
            if (i0 + i < cnt) block(bl[i], wb0 + i0 + i);
        }
      }
    }
    __syncthreads();  // the next round overwrites the staged slice
  }

  // D[4q + v][nl]: y partials per (m, n) and u partials per (m, j)
#pragma unroll
  for (int v = 0; v < 4; ++v) red[wave][4 * q + v][nl] = acc[v];
#pragma unroll
  for (int jt = 0; jt < JT; ++jt)
#pragma unroll
    for (int v = 0; v < 4; ++v) ured[wave][4 * q + v][16 * jt + nl] = (JT == 1 ? uacc[jt][v] + uacc1[0][v] : uacc[jt][v]);
  __syncthreads();
  if (part) {
    // split contraction: this split's sums over its rounds, the bypass term
    // added by k_gemv_reduce.  part = y partials [S][M][N], then u partials
    // [S][M][r] (every row group computes the same u; the first stores it).
    const int64_t sp = blockIdx.y;
    if (blockIdx.x == 0) {
      float *pu = part + (int64_t)gridDim.y * M * N;
      for (int e = t; e < 16 * 16 * JT; e += kGemvThreads) {
        const int mo = e / (16 * JT), j = e % (16 * JT);
        float su = 0.0f;
#pragma unroll
        for (int w = 0; w < kGemvWaves; ++w) su += ured[w][mo][j];
        if (mo < M && j < r) pu[(sp * M + mo) * r + j] = su;
      }
    }
    if (t < 256) {
      const int mo = t >> 4, no = t & 15;
      const int64_t nn = n0 + no;
      if (mo < M && nn < N) {
        float sum = 0.0f;
#pragma unroll
        for (int w = 0; w < kGemvWaves; ++w) sum += red[w][mo][no];
        part[(sp * M + mo) * N + nn] = sum;
      }
    }
    return;
  }
  for (int e = t; e < 16 * 16 * JT; e += kGemvThreads) {
    const int mo = e / (16 * JT), j = e % (16 * JT);
    float su = 0.0f;
#pragma unroll
    for (int w = 0; w < kGemvWaves; ++w) su += ured[w][mo][j];
    us[mo][j] = su;
    if (u_save && blockIdx.x == 0 && mo < M && j < r) u_save[mo * r + j] = su;
  }
  __syncthreads();
  if (t < 256) {
    const int mo = t >> 4, no = t & 15;
    const int64_t nn = n0 + no;
    if (mo < M && nn < N) {
      float sum = 0.0f;
#pragma unroll
      for (int w = 0; w < kGemvWaves; ++w) sum += red[w][mo][no];
      float l = 0.0f;
      for (int j = 0; j < r; ++j) l = __builtin_fmaf(us[mo][j], bs[no][j], l);
      y[(int64_t)mo * N + nn] = Half<AT>::bits(__builtin_fmaf(s, l, sum));
    }
  }
}

// The contraction splits of k_gemv_fwd summed in split order, then the
// bypass term, as the single-split epilogue forms it: u[m][j] = sum over
// splits, y[m][n] = RN(fmaf(s, sum_j u[m][j] B[n][j], sum over splits)).
// Grid (ceil(N / 256), M); the first column of workgroups stores u_save.
template <typename AT, typename LT>
__global__ __launch_bounds__(256) void k_gemv_reduce(const float *__restrict__ part, int S, int M,
                                                     int64_t N, int32_t r,
                                                     const LT *__restrict__ B, float s,
                                                     uint16_t *__restrict__ y,
                                                     float *__restrict__ u_save) {
  __shared__ float us[128];
  const int m = blockIdx.y, t = threadIdx.x;
  const float *pu = part + (int64_t)S * M * N;
  if (t < r) {
    float su = 0.0f;
    for (int sp = 0; sp < S; ++sp) su += pu[((int64_t)sp * M + m) * r + t];
    us[t] = su;
    if (u_save && blockIdx.x == 0) u_save[(int64_t)m * r + t] = su;
  }
  __syncthreads();
  const int64_t n = (int64_t)blockIdx.x * 256 + t;
  if (n >= N) return;
  float sum = 0.0f;
  for (int sp = 0; sp < S; ++sp) sum += part[((int64_t)sp * M + m) * N + n];
  float l = 0.0f;
  for (int j = 0; j < r; ++j) l = __builtin_fmaf(us[j], load_as_f32(B, n * r + j), l);
  y[(int64_t)m * N + n] = Half<AT>::bits(__builtin_fmaf(s, l, sum));
}

template <typename AT, typename LT, int JT, int XM, int WPE = 2>
static void launch_xm(dim3 grid, hipStream_t stream, const uint16_t *x, int M,
                      const uint8_t *packed, BlockScales sc, int64_t N, int64_t K, const void *A,
                      const void *B, int32_t r, float s, uint16_t *y, float *u_save, float *part) {
  if (sc.absmax == nullptr)
    hipLaunchKernelGGL((k_gemv_fwd<AT, LT, JT, true, XM, WPE>), grid, dim3(kGemvThreads), 0,
                       stream, x, M, packed, sc, N, K, (const LT *)A, (const LT *)B, r, s, y,
                       u_save, part);
  else
    hipLaunchKernelGGL((k_gemv_fwd<AT, LT, JT, false, XM, WPE>), grid, dim3(kGemvThreads), 0,
                       stream, x, M, packed, sc, N, K, (const LT *)A, (const LT *)B, r, s, y,
                       u_save, part);
}

// Compute units of the chip (MI355X): a grid larger than this runs in
// several rounds of workgroups per unit.
constexpr unsigned kGemvUnits = 256;

template <typename AT, typename LT, int JT>
static void launch_jt(dim3 grid, hipStream_t stream, const uint16_t *x, int M,
                      const uint8_t *packed, BlockScales sc, int64_t N, int64_t K, const void *A,
                      const void *B, int32_t r, float s, uint16_t *y, float *u_save,
                      float *part) {
  // More workgroups than units, and a footprint two of which fit a unit's
  // LDS (rank tiles of 16 or 32, activations staged for one token row or
  // read in operand layout): two workgroups per unit.  For 2-4 token rows
  // the one-per-unit form with the rows staged in LDS is faster (14336 x
  // 4096 weight, 4 rows: 27 against 32 us).
  if constexpr (JT <= 2) {
    if (grid.x * grid.y > kGemvUnits && (M == 1 || M > 4)) {
      if (M == 1)
        launch_xm<AT, LT, JT, 1, 4>(grid, stream, x, M, packed, sc, N, K, A, B, r, s, y, u_save, part);
      else
        launch_xm<AT, LT, JT, 0, 4>(grid, stream, x, M, packed, sc, N, K, A, B, r, s, y, u_save, part);
      return;
    }
  }
  if (M == 1)
    launch_xm<AT, LT, JT, 1>(grid, stream, x, M, packed, sc, N, K, A, B, r, s, y, u_save, part);
  else if (M <= 4)
    launch_xm<AT, LT, JT, 4>(grid, stream, x, M, packed, sc, N, K, A, B, r, s, y, u_save, part);
  else
    launch_xm<AT, LT, JT, 0>(grid, stream, x, M, packed, sc, N, K, A, B, r, s, y, u_save, part);
}

template <typename AT, typename LT>
static void launch_lt(dim3 grid, hipStream_t stream, const uint16_t *x, int M,
                      const uint8_t *packed, BlockScales sc, int64_t N, int64_t K, const void *A,
                      const void *B, int32_t r, float s, uint16_t *y, float *u_save,
                      float *part) {
  if (r <= 16) launch_jt<AT, LT, 1>(grid, stream, x, M, packed, sc, N, K, A, B, r, s, y, u_save, part);
  else if (r <= 32) launch_jt<AT, LT, 2>(grid, stream, x, M, packed, sc, N, K, A, B, r, s, y, u_save, part);
  else if (r <= 64) launch_jt<AT, LT, 4>(grid, stream, x, M, packed, sc, N, K, A, B, r, s, y, u_save, part);
  else launch_jt<AT, LT, 8>(grid, stream, x, M, packed, sc, N, K, A, B, r, s, y, u_save, part);
}

// Workgroups a split contraction aims for: two per compute unit.
constexpr int64_t kGemvSplitTarget = 2 * kGemvUnits;

// Contraction splits of a decode forward: one unless the row groups leave
// at least half the units idle and there are rounds to share; no split is
// left without rounds.  (At 129-256 groups the split's second launch and the
// smaller register budget cost more than it gains: 4096 x 14336 weight, one
// token, 23.4 us unsplit against 26.7 split in 2; at 64 groups, 1024 x 14336,
// 21.0 against 12.6 split in 4.)
static int gemv_splits(int64_t N, int64_t K) {
  const int64_t groups = (N + kGemvRows - 1) / kGemvRows;
  const int64_t rounds = ((K >> 6) + kGemvRound - 1) / kGemvRound;
  if (rounds < 2 || 2 * groups > kGemvUnits) return 1;
  int64_t S = (kGemvSplitTarget + groups - 1) / groups;
  if (S > rounds) S = rounds;
  if (S < 2) return 1;
  const int64_t per = (rounds + S - 1) / S;
  return (int)((rounds + per - 1) / per);
}

size_t gemv_fwd_partial_floats(int64_t M, int64_t N, int64_t K, int32_t r) {
  const int S = gemv_splits(N, K);
  return S > 1 ? (size_t)S * M * (N + r) : 0;
}

// A 16-bit LoRA factor has the activations' format (checked by the caller).
int launch_gemv_fwd(const void *xv, int act_dtype, int64_t M, const uint8_t *packed,
                    BlockScales sc, int64_t N, int64_t K, const void *A, const void *B,
                    int lora_dtype, int32_t r, float s, void *yv, float *u_save,
                    hipStream_t stream, float *part) {
  const uint16_t *x = (const uint16_t *)xv;
  uint16_t *y = (uint16_t *)yv;
  const int S = part ? gemv_splits(N, K) : 1;
  const dim3 grid((unsigned)((N + kGemvRows - 1) / kGemvRows), (unsigned)S);
  float *p = S > 1 ? part : nullptr;
  with_half(act_dtype, [&](auto *tag) {
    using AT = elem_of<decltype(tag)>;
    if (lora_dtype == QL_F32)
      launch_lt<AT, float>(grid, stream, x, (int)M, packed, sc, N, K, A, B, r, s, y, u_save, p);
    else
      launch_lt<AT, AT>(grid, stream, x, (int)M, packed, sc, N, K, A, B, r, s, y, u_save, p);
    if (S > 1) {
      const dim3 rgrid((unsigned)((N + 255) / 256), (unsigned)M);
      if (lora_dtype == QL_F32)
        hipLaunchKernelGGL((k_gemv_reduce<AT, float>), rgrid, dim3(256), 0, stream, p, S, (int)M,
                           N, r, (const float *)B, s, y, u_save);
      else
        hipLaunchKernelGGL((k_gemv_reduce<AT, AT>), rgrid, dim3(256), 0, stream, p, S, (int)M,
                           N, r, (const AT *)B, s, y, u_save);
    }
  });
  QL_HIP_CHECK_LAUNCH();
  return QL_OK;
}

}  // namespace qlora
