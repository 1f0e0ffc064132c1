// gemm.hip -- matrix-core (16-bit MFMA, fp32 accumulate) products of the
// QLoRA layer for many tokens:
//
//   forward:        y  = x W^^T + s u B^T   (26. QLoRA and 4bit Quantization, Step 3)
//   input gradient: dx = dy W^  + g A       (22. QLoRA and 4bit Quantization, Step 1:
//                                            the gradient flows through the frozen base)
//
// W^ is never materialised: each workgroup dequantises the NF4 tile it needs
// (26. ..., Step 4: table[index] * scale; 22. ..., Step 3: restored to a 16-bit
// float for the product) straight into LDS in the compute format and feeds
// the matrix cores from there.  The compute format is the activations'
// 16-bit format AT (bf16, or fp16: Gemma lesson 09, sec. 9.3, compute
// dtype); every kernel is written once for both through Half<AT>.  The
// rank-r bypass is folded into the same accumulators as extra 16-deep MFMA
// steps (u and g are fp32 in memory and are rounded to AT for those steps).
//
// Tiles: 256 tokens x BN outputs per workgroup (BN = 256 or 128), contraction
// step 64 (= one 64-element chunk of every weight row in the forward: one
// NF4 block, or half of one with blocks of 128), 8 waves laid
// out 2 (tokens) x 4 (outputs), each owning a 128 x BN/4 block of 32x32
// accumulator tiles.  LDS is double-buffered: while the matrix cores work on
// step k, the registers loaded during step k-1 (step k+1's tiles) are written
// to the other buffer and step k+2's global loads are issued; one barrier
// per step.  LDS rows are 64 16-bit values = 8 chunks of 16 bytes.  gfx950 serves a
// 16-byte-per-lane LDS read 16 lanes per pass over 64 banks (256 bytes), so
// the 16 rows one pass touches must land on 16 distinct 16-byte bank slots:
// chunk c of row r is stored at position c ^ ((r >> 1) & 7); with the row
// parity choosing the bank half this spreads any 16 consecutive rows read at
// the same logical chunk over all 64 banks.
//
// v_mfma_f32_32x32x16_{bf16,f16} layout (gfx950): A lane l holds A[l % 32][8*(l/32)
// .. +8], B lane l holds B[8*(l/32) .. +8][l % 32], result register v of lane
// l is D[8*(v/4) + 4*(l/32) + v%4][l % 32].
//
// The matrix cores compute the transposed output tile (weight operand as A,
// activation operand as B), so that each lane ends with runs of 4
// consecutive output columns of one row and stores them as 8-byte words.
// The rank-r bypass is accumulated first, before the main loop, so the loads
// of its operands overlap the loads of the first tiles.
#include "kernels.h"
#include "upart.h"

namespace qlora {

constexpr int kBM = 256;
constexpr int kBK = 64;
constexpr int kThreads = 512;
constexpr int kRowBytes = 128;  // 64 16-bit values per LDS row

__device__ __forceinline__ int swz(int row, int chunk) {
  return row * kRowBytes + ((chunk ^ ((row >> 1) & 7)) << 4);
}

template <typename AT>
__device__ __forceinline__ f32x16 mfma32(const u32x4 &a, const u32x4 &b, const f32x16 &c) {
  return Half<AT>::mfma32(a, b, c);
}

// Workgroup -> tile.  Consecutive workgroup ids are spread round-robin over
// the 8 XCDs; remap so that each XCD receives a contiguous range of logical
// tiles.  Logical tiles go in groups of two token tiles: within a group the
// token tile alternates fastest, then the output column.  An XCD thus works
// on a 2 x (its share of columns) block: its two activation strips stay in
// its L2, and each weight tile is read by two workgroups at about the same
// time (one L2 miss instead of two), which halves the weight traffic
// compared with giving each XCD whole rows of tiles.
__device__ __forceinline__ void tile_of(int64_t mt_count, int64_t nt_count, int64_t &mt,
                                        int64_t &nt) {
  const int64_t G = mt_count * nt_count;
  const int64_t bid = blockIdx.x;
  const int64_t L = (G % 8 == 0) ? (bid % 8) * (G / 8) + bid / 8 : bid;
  if (mt_count % 2 == 0) {
    const int64_t grp = L / (2 * nt_count), i = L % (2 * nt_count);
    mt = grp * 2 + (i & 1);
    nt = i >> 1;
  } else {
    mt = L / nt_count;
    nt = L % nt_count;
  }
}

// 256 rows x 64 16-bit activation tile in registers: 4 chunks of 16 B per lane.
struct ActStage {
  u32x4 v[4];
};

__device__ __forceinline__ void zero_acc(f32x16 *acc, int n) {
  for (int i = 0; i < n; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[i][v] = 0.0f;
}

// Store a wave's transposed accumulators in format AT: register v of
// accumulator (i, j) in lane l is out[row][col], row = row_base + 32 i +
// l % 32, col = col_base + 32 j + 8 (v / 4) + 4 (l / 32) + v % 4.  Full
// tiles use 8-byte stores; a tile crossing the last column stores element
// by element.
template <typename AT, int MI, int NJ>
__device__ __forceinline__ void store_tile_t(uint16_t *__restrict__ out, int64_t ld, int64_t rows,
                                             int64_t cols, int64_t row_base, int64_t col_base,
                                             const f32x16 (&acc)[MI][NJ], int lane) {
  const int lr = lane & 31, lk = lane >> 5;
  const bool full = col_base + 32 * NJ <= cols && ld % 4 == 0;
#pragma unroll
  for (int i = 0; i < MI; ++i) {
    const int64_t m = row_base + 32 * i + lr;
    if (m >= rows) continue;
    uint16_t *p = out + m * ld + col_base + 4 * lk;
    if (full) {
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          *reinterpret_cast<u32x2 *>(p + 32 * j + 8 * q) =
              u32x2{Half<AT>::pack2(acc[i][j][4 * q], acc[i][j][4 * q + 1]),
                    Half<AT>::pack2(acc[i][j][4 * q + 2], acc[i][j][4 * q + 3])};
    } else {
      for (int j = 0; j < NJ; ++j)
        for (int v = 0; v < 16; ++v) {
          const int c = 32 * j + 8 * (v >> 2) + (v & 3);
          if (col_base + 4 * lk + c < cols) p[c] = Half<AT>::bits(acc[i][j][v]);
        }
    }
  }
}

// Store a wave's transposed accumulators as fp32 (a split-K partial tile):
// 4 consecutive columns per 16-byte store when ld % 4 == 0 and the tile is
// full, else element by element.
template <int MI, int NJ>
__device__ __forceinline__ void store_tile_f32(float *__restrict__ out, int64_t ld, int64_t rows,
                                               int64_t cols, int64_t row_base, int64_t col_base,
                                               const f32x16 (&acc)[MI][NJ], int lane) {
  const int lr = lane & 31, lk = lane >> 5;
  const bool full = col_base + 32 * NJ <= cols && ld % 4 == 0;
#pragma unroll
  for (int i = 0; i < MI; ++i) {
    const int64_t m = row_base + 32 * i + lr;
    if (m >= rows) continue;
    float *p = out + m * ld + col_base + 4 * lk;
    if (full) {
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          *reinterpret_cast<f32x4 *>(p + 32 * j + 8 * q) =
              f32x4{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                    acc[i][j][4 * q + 3]};
    } else {
      for (int j = 0; j < NJ; ++j)
        for (int v = 0; v < 16; ++v) {
          const int c = 32 * j + 8 * (v >> 2) + (v & 3);
          if (col_base + 4 * lk + c < cols) p[c] = acc[i][j][v];
        }
    }
  }
}

// out[e] = AT(sum_s part[s][e]), s in increasing order; 4 elements per lane
// (count % 4 == 0).
template <typename AT>
__global__ __launch_bounds__(256) void k_reduce_split(const float *__restrict__ part, int S,
                                                      int64_t count, uint16_t *__restrict__ out) {
  const int64_t e = 4 * ((int64_t)blockIdx.x * 256 + threadIdx.x);
  if (e >= count) return;
  f32x4 acc = *reinterpret_cast<const f32x4 *>(part + e);
  for (int i = 1; i < S; ++i) {
    const f32x4 v = *reinterpret_cast<const f32x4 *>(part + (int64_t)i * count + e);
    acc = f32x4{acc[0] + v[0], acc[1] + v[1], acc[2] + v[2], acc[3] + v[3]};
  }
  *reinterpret_cast<u32x2 *>(out + e) =
      u32x2{Half<AT>::pack2(acc[0], acc[1]), Half<AT>::pack2(acc[2], acc[3])};
}

// Rank-r operand tiles are staged once per 16-rank chunk into LDS in format AT
// rows of 16 values with a 48-byte stride (the 16 rows one 16-byte-per-lane
// read pass touches then start on 16 distinct 4-bank groups).
constexpr int kLoraStride = 48;

// rows x 16 slice [j0, j0 + 16) of a row-major [*, r] factor, times scale,
// rounded to AT; rows past `valid` and ranks past r are zero.
template <int ROWS, int NT, typename AT, typename T>
__device__ __forceinline__ void stage_lora(uint8_t *dst, const T *__restrict__ src, int64_t row0,
                                           int64_t valid, int32_t r, int j0, float scale, int t) {
  for (int e = t; e < ROWS * 16; e += NT) {
    const int row = e >> 4, jj = e & 15;
    const int64_t gr = row0 + row;
    float v = 0.0f;
    if (gr < valid && j0 + jj < r) v = scale * load_as_f32(src, gr * r + j0 + jj);
    *reinterpret_cast<uint16_t *>(dst + row * kLoraStride + 2 * jj) = Half<AT>::bits(v);
  }
}

// ROWS x 16 slice of the transpose of a row-major [r, ld] factor: staged
// row `row` holds src[(j0 + jj) * ld + col0 + row], jj = 0..15 (lanes walk
// along a source row, so the loads are coalesced); columns past ld and
// ranks past r are zero.
template <int ROWS, int NT, typename AT, typename T>
__device__ __forceinline__ void stage_lora_t(uint8_t *dst, const T *__restrict__ src, int64_t ld,
                                             int64_t col0, int32_t r, int j0, int t) {
  for (int e = t; e < ROWS * 16; e += NT) {
    const int jj = e / ROWS, row = e % ROWS;
    float v = 0.0f;
    if (j0 + jj < r && col0 + row < ld) v = load_as_f32(src, (int64_t)(j0 + jj) * ld + col0 + row);
    *reinterpret_cast<uint16_t *>(dst + row * kLoraStride + 2 * jj) = Half<AT>::bits(v);
  }
}

__device__ __forceinline__ u32x4 lora_frag(const uint8_t *src, int row, int lk) {
  return *reinterpret_cast<const u32x4 *>(src + row * kLoraStride + 16 * lk);
}

// Write a wave's transposed accumulators (see store_tile_t) through a
// wave-private LDS slice of 32 rows, so every global store instruction
// writes whole 16-byte pieces of 64 / (TN / 8) consecutive rows.  Needs a
// full tile in the column direction and ld % 8 == 0.
template <typename AT, int MI, int NJ>
__device__ __forceinline__ void store_tile_lds(uint16_t *__restrict__ out, int64_t ld,
                                               int64_t rows, int64_t row_base, int64_t col_base,
                                               const f32x16 (&acc)[MI][NJ], uint8_t *slice,
                                               int lane) {
  constexpr int TN = 32 * NJ;
  constexpr int OS = 2 * TN + 16;   // bytes per staged row
  constexpr int CPR = TN / 8;       // 16-byte pieces per row
  constexpr int RPI = 64 / CPR;     // rows per store instruction
  const int lr = lane & 31, lk = lane >> 5;
#pragma unroll
  for (int i = 0; i < MI; ++i) {
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *reinterpret_cast<u32x2 *>(slice + lr * OS + 2 * (32 * j + 8 * q + 4 * lk)) =
            u32x2{Half<AT>::pack2(acc[i][j][4 * q], acc[i][j][4 * q + 1]),
                  Half<AT>::pack2(acc[i][j][4 * q + 2], acc[i][j][4 * q + 3])};
#pragma unroll
    for (int it = 0; it < 32 / RPI; ++it) {
      const int row = it * RPI + lane / CPR, c = lane % CPR;
      const u32x4 v = *reinterpret_cast<const u32x4 *>(slice + row * OS + 16 * c);
      const int64_t m = row_base + 32 * i + row;
      if (m < rows) *reinterpret_cast<u32x4 *>(out + m * ld + col_base + 8 * c) = v;
    }
  }
}

// ===========================================================================
// Forward
// ===========================================================================
template <int BN, typename AT, typename LT, bool DQ>
__global__ __launch_bounds__(kThreads) void k_gemm_fwd(const uint16_t *__restrict__ x, int64_t M,
                                                       const uint8_t *__restrict__ packed,
                                                       BlockScales sc, int64_t N, int64_t K,
                                                       const float *__restrict__ u,
                                                       const LT *__restrict__ B, int32_t r,
                                                       float s, uint16_t *__restrict__ y,
                                                       float *__restrict__ part, int nsplit) {
  constexpr int TN = BN / 4;           // outputs per wave
  constexpr int NJ = TN / 32;          // 32-wide tiles per wave along outputs
  constexpr int WBYTES = BN * 32 / kThreads;  // packed bytes per lane per step (16 or 8)
  constexpr int LPR = 32 / WBYTES;            // lanes per weight row
  __shared__ __attribute__((aligned(16))) uint8_t xs[2][kBM * kRowBytes];
  __shared__ __attribute__((aligned(16))) uint8_t ws[2][BN * kRowBytes];
  __shared__ __attribute__((aligned(16))) uint8_t ls_u[kBM * kLoraStride];
  __shared__ __attribute__((aligned(16))) uint8_t ls_b[BN * kLoraStride];
  __shared__ float2 lut[256];
  const int t = threadIdx.x;
  if (t < 256) lut[t] = make_float2(c_nf4[t >> 4], c_nf4[t & 15]);

  int64_t mt, nt;
  tile_of((M + kBM - 1) / kBM, (N + BN - 1) / BN, mt, nt);
  const int64_t m0 = mt * kBM, n0 = nt * BN;
  const int64_t KB = K >> 6;
  // contraction slice of this workgroup (split-K: grid row blockIdx.y)
  const int split = blockIdx.y;
  const int ks0 = (int)(split * KB / nsplit), ks1 = (int)((split + 1) * KB / nsplit);

  // weight staging: lane -> (row, part) of the packed tile.  Rows past N
  // (and token rows past M below) are clamped to the last valid row instead
  // of predicated: they only feed outputs that are never stored, and
  // branch-free loads let the compiler count outstanding loads exactly.
  const int w_row = t / LPR, w_part = t % LPR;
  const int64_t w_n = n0 + w_row < N ? n0 + w_row : N - 1;
  const uint8_t *w_src = packed + ((w_n * K) >> 1) + WBYTES * w_part;
  const int64_t w_sc = w_n * KB;

  const float mu = DQ ? sc.mu[0] : 0.0f;

  ActStage xr;
  uint32_t wr[WBYTES / 4];
  // the block constant travels as its raw parts (code and sigma, or the fp32
  // absmax) and is combined only when the tile is staged, so that no wait
  // for the just-issued prefetch is needed
  int wq = 0;
  float wsig = 0.0f;
  auto load_w = [&](int step) {
    if constexpr (WBYTES == 16) {
      const u32x4 v = *reinterpret_cast<const u32x4 *>(w_src + 32 * (int64_t)step);
      wr[0] = v.x; wr[1] = v.y; wr[2] = v.z; wr[3] = v.w;
    } else {
      const u32x2 v = *reinterpret_cast<const u32x2 *>(w_src + 32 * (int64_t)step);
      wr[0] = v.x; wr[1] = v.y;
    }
    const int64_t b = sc.index(w_sc + step);
    if constexpr (DQ) {
      wq = sc.q[b];
      wsig = sc.sigma[b >> 8];
    } else {
      wsig = sc.absmax[b];
    }
  };
  const uint16_t *x_src[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int id = t + kThreads * i;
    const int64_t rr = m0 + (id >> 3) < M ? m0 + (id >> 3) : M - 1;
    x_src[i] = x + rr * K + 8 * (id & 7);
  }
  auto load_x_chunk = [&](int step, int i) {
    xr.v[i] = *reinterpret_cast<const u32x4 *>(x_src[i] + (int64_t)step * kBK);
  };
  // quarter q of the staging of one step into LDS buffer buf: activation
  // chunk q and the q-th quarter of this lane's dequantised weight bytes
  auto store_quarter = [&](int buf, int qq) {
    const int id = t + kThreads * qq;
    *reinterpret_cast<u32x4 *>(xs[buf] + swz(id >> 3, id & 7)) = xr.v[qq];
    const float wa = DQ ? __builtin_fmaf((float)wq, wsig, mu) : wsig;
    constexpr int BPQ = WBYTES / 4;  // packed bytes per quarter: 4 or 2
    uint32_t d[BPQ];
#pragma unroll
    for (int e = 0; e < BPQ; ++e) {
      const int bi = BPQ * qq + e;
      const float2 p = lut[(wr[bi >> 2] >> (8 * (bi & 3))) & 0xFF];
      d[e] = Half<AT>::pack2(p.x * wa, p.y * wa);
    }
    if constexpr (BPQ == 4) {
      *reinterpret_cast<u32x4 *>(ws[buf] + swz(w_row, 4 * w_part + qq)) =
          u32x4{d[0], d[1], d[2], d[3]};
    } else {
      // 8-byte halves of the lane's two 16-byte chunks
      *reinterpret_cast<u32x2 *>(ws[buf] + swz(w_row, 2 * w_part + (qq >> 1)) + 8 * (qq & 1)) =
          u32x2{d[0], d[1]};
    }
  };

  const int wave = t >> 6, lane = t & 63;
  const int wm = wave & 1, wn = wave >> 1;
  const int lr = lane & 31, lk = lane >> 5;
  f32x16 acc[4][NJ];
  zero_acc(&acc[0][0], 4 * NJ);

  __syncthreads();  // lut
#pragma unroll
  for (int i = 0; i < 4; ++i) load_x_chunk(ks0, i);
  load_w(ks0);
  // first 16-rank chunk of the bypass operands (s u and B), used after the
  // main loop by the first contraction slice; staged here so that its loads
  // overlap the first tile loads
  if (split == 0) {
    stage_lora<kBM, kThreads, AT>(ls_u, u, m0, M, r, 0, s, t);
    stage_lora<BN, kThreads, AT>(ls_b, B, n0, N, r, 0, 1.0f, t);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) store_quarter(0, i);
#pragma unroll
  for (int i = 0; i < 4; ++i) load_x_chunk(ks0 + 1 < ks1 ? ks0 + 1 : ks0, i);
  load_w(ks0 + 1 < ks1 ? ks0 + 1 : ks0);
  __syncthreads();
  // The staging of step k+1 and the prefetch of step k+2 run unconditionally
  // (clamped to the last step): the extra work in the last two iterations
  // writes a buffer no one reads again and keeps the loop free of branches.
  for (int k = ks0; k < ks1; ++k) {
    const int cur = (k - ks0) & 1;
    const int pf = k + 2 < ks1 ? k + 2 : ks1 - 1;
    const uint8_t *xb = xs[cur];
    const uint8_t *wb = ws[cur];
    u32x4 a[2][4], b[2][NJ];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      a[0][i] = *reinterpret_cast<const u32x4 *>(xb + swz(128 * wm + 32 * i + lr, lk));
#pragma unroll
    for (int j = 0; j < NJ; ++j)
      b[0][j] = *reinterpret_cast<const u32x4 *>(wb + swz(TN * wn + 32 * j + lr, lk));
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int cb = kk & 1, nb = cb ^ 1;
      if (kk < 3) {
        const int chunk = 2 * (kk + 1) + lk;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          a[nb][i] = *reinterpret_cast<const u32x4 *>(xb + swz(128 * wm + 32 * i + lr, chunk));
#pragma unroll
        for (int j = 0; j < NJ; ++j)
          b[nb][j] = *reinterpret_cast<const u32x4 *>(wb + swz(TN * wn + 32 * j + lr, chunk));
      }
      store_quarter(cur ^ 1, kk);
      load_x_chunk(pf, kk);
      if (kk == 3) load_w(pf);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j) acc[i][j] = mfma32<AT>(b[cb][j], a[cb][i], acc[i][j]);
    }
    __syncthreads();
  }

  // LoRA bypass: acc += B (s u)^T, 16 ranks per MFMA step (the main loop's
  // last barrier orders the staged chunk 0 before these reads); only the
  // first contraction slice adds it.
  for (int j0 = 0; j0 < (split == 0 ? r : 0); j0 += 16) {
    if (j0 > 0) {
      __syncthreads();
      stage_lora<kBM, kThreads, AT>(ls_u, u, m0, M, r, j0, s, t);
      stage_lora<BN, kThreads, AT>(ls_b, B, n0, N, r, j0, 1.0f, t);
      __syncthreads();
    }
    u32x4 ua[4], bb[NJ];
#pragma unroll
    for (int i = 0; i < 4; ++i) ua[i] = lora_frag(ls_u, 128 * wm + 32 * i + lr, lk);
#pragma unroll
    for (int j = 0; j < NJ; ++j) bb[j] = lora_frag(ls_b, TN * wn + 32 * j + lr, lk);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j) acc[i][j] = mfma32<AT>(bb[j], ua[i], acc[i][j]);
  }
  if (nsplit > 1)
    store_tile_f32<4, NJ>(part + (int64_t)split * M * N, N, M, N, m0 + 128 * wm, n0 + TN * wn, acc,
                       lane);
  else if (n0 + BN <= N && N % 8 == 0)
    store_tile_lds<AT, 4, NJ>(y, N, M, m0 + 128 * wm, n0 + TN * wn, acc,
                       &xs[0][0] + wave * 32 * (2 * TN + 16), lane);
  else
    store_tile_t<AT, 4, NJ>(y, N, M, N, m0 + 128 * wm, n0 + TN * wn, acc, lane);
}

// ===========================================================================
// Forward for few tokens (up to a few hundred): BM = 64 or 128 tokens x 128
// outputs per workgroup, 4 waves, wave w owning outputs 32 w .. 32 w + 31
// for all BM tokens.  A 256-token tile would run the matrix cores mostly on
// padding rows, and with one wave per output row the weight tile needs no
// dequantised copy in LDS: it is staged as packed codes (4 KB per step)
// plus one block constant per row, and every wave dequantises its own rows
// in registers right before its matrix ops, once for all BM tokens (the
// 128-token tile halves the weight reads and the dequantisation per token
// of the 64-token one).
//
// The contraction order inside a step is permuted so that a lane's 16
// packed bytes (32 consecutive codes of one row) feed all four 16-deep
// matrix ops of the step: for op kk, lane half h = l / 32 covers
// k = 32 h + 8 kk + 0..7 in both operands (the weight from registers, the
// activations from LDS chunk 4 h + kk of the token row).
// ===========================================================================
constexpr int kSmBM = 64;   // token tile of the fused form and of the smallest calls
constexpr int kSmBN = 128;
constexpr int kSmThreads = 256;

//
// FUSED: the launch also computes u and leaves the bypass to the launch that
// sums its partials.  Workgroups past the G tiles (grid row 0 only; the
// others return) each form one u slice tile -- token group, rank tile and
// contraction slice -- from x and A; every tile workgroup writes its fp32
// partial of x W^^T for its contraction slice (no bypass), and the next
// launch forms y = RN(fmaf(s, sum_j u_j B_nj, sum of the slices)).
template <int BM, typename AT, typename LT, bool DQ, bool FUSED>
__global__ __launch_bounds__(kSmThreads) void k_gemm_fwd_small(
    const uint16_t *__restrict__ x, int64_t M, const uint8_t *__restrict__ packed, BlockScales sc,
    int64_t N, int64_t K, const float *__restrict__ u, const LT *__restrict__ B, int32_t r,
    float s, uint16_t *__restrict__ y, float *__restrict__ part, int nsplit,
    const LT *__restrict__ A, float *__restrict__ upart, int uc, int MT, Dropout dr) {
  static_assert(BM == 64 || BM == 128, "token tiles of 64 or 128");
  constexpr int MI = BM / 32;                // 32-token MFMA tiles per wave
  constexpr int XR = BM * 8 / kSmThreads;    // 16-byte activation chunks per lane per step
  __shared__ __attribute__((aligned(16))) uint8_t xs[2][BM * kRowBytes];
  __shared__ __attribute__((aligned(16))) uint8_t wp[2][kSmBN * 32];
  __shared__ float wsc[2][kSmBN];
  __shared__ __attribute__((aligned(16))) uint8_t ls_u[BM * kLoraStride];
  __shared__ __attribute__((aligned(16))) uint8_t ls_b[kSmBN * kLoraStride];
  __shared__ float2 lut[256];
  const int t = threadIdx.x;
  const int64_t G = ((M + BM - 1) / BM) * ((N + kSmBN - 1) / kSmBN);
  if (FUSED && (int64_t)blockIdx.x >= G) {
    if (blockIdx.y == 0) {
      const int JT = (r + 15) / 16;
      const int b = (int)((int64_t)blockIdx.x - G);
      u_slice_tile<AT, LT>(x, (int)M, K, A, r, upart, uc, b / (JT * MT), (b / MT) % JT, b % MT,
                           reinterpret_cast<float *>(&xs[0][0]), dr);
    }
    return;
  }
  lut[t] = make_float2(c_nf4[t >> 4], c_nf4[t & 15]);

  int64_t mt, nt;
  tile_of((M + BM - 1) / BM, (N + kSmBN - 1) / kSmBN, mt, nt);
  const int64_t m0 = mt * BM, n0 = nt * kSmBN;
  const int64_t KB = K >> 6;
  const int split = blockIdx.y;
  const int ks0 = (int)(split * KB / nsplit), ks1 = (int)((split + 1) * KB / nsplit);

  // staging: lane t stages half t & 1 (16 bytes) of weight row t >> 1 and
  // activation chunks t + 256 i, i < XR (token rows 32 i + (t >> 3)); rows
  // past N or M are clamped to the last valid row (their outputs are never
  // stored)
  const int w_row = t >> 1, w_half = t & 1;
  const int64_t w_n = n0 + w_row < N ? n0 + w_row : N - 1;
  const uint8_t *w_src = packed + ((w_n * K) >> 1) + 16 * w_half;
  const int64_t w_sc = w_n * KB;
  const float mu = DQ ? sc.mu[0] : 0.0f;
  const uint16_t *x_src[XR];
#pragma unroll
  for (int i = 0; i < XR; ++i) {
    const int id = t + kSmThreads * i;
    const int64_t rr = m0 + (id >> 3) < M ? m0 + (id >> 3) : M - 1;
    x_src[i] = x + rr * K + 8 * (id & 7);
  }
  u32x4 xr[XR], wr;
  int wq = 0;
  float wsig = 0.0f;
  auto load_x = [&](int step, int i) {
    xr[i] = *reinterpret_cast<const u32x4 *>(x_src[i] + (int64_t)step * kBK);
  };
  auto load_w = [&](int step) {
    wr = *reinterpret_cast<const u32x4 *>(w_src + 32 * (int64_t)step);
    const int64_t b = sc.index(w_sc + step);
    if constexpr (DQ) {
      wq = sc.q[b];
      wsig = sc.sigma[b >> 8];
    } else {
      wsig = sc.absmax[b];
    }
  };
  auto store_x = [&](int buf, int i) {
    const int id = t + kSmThreads * i;
    *reinterpret_cast<u32x4 *>(xs[buf] + swz(id >> 3, id & 7)) = xr[i];
  };
  auto store_w = [&](int buf) {
    *reinterpret_cast<u32x4 *>(wp[buf] + 32 * w_row + 16 * w_half) = wr;
    if (w_half == 0) wsc[buf][w_row] = DQ ? __builtin_fmaf((float)wq, wsig, mu) : wsig;
  };

  const int wave = t >> 6, lane = t & 63;
  const int lr = lane & 31, lk = lane >> 5;
  const int my_row = 32 * wave + lr;  // this lane's weight row in the tile
  f32x16 acc[MI][1];
  zero_acc(&acc[0][0], MI);

  __syncthreads();  // lut
#pragma unroll
  for (int i = 0; i < XR; ++i) load_x(ks0, i);
  load_w(ks0);
  if (!FUSED && split == 0) {
    stage_lora<BM, kSmThreads, AT>(ls_u, u, m0, M, r, 0, s, t);
    stage_lora<kSmBN, kSmThreads, AT>(ls_b, B, n0, N, r, 0, 1.0f, t);
  }
#pragma unroll
  for (int i = 0; i < XR; ++i) store_x(0, i);
  store_w(0);
  {
    const int nx = ks0 + 1 < ks1 ? ks0 + 1 : ks0;
#pragma unroll
    for (int i = 0; i < XR; ++i) load_x(nx, i);
    load_w(nx);
  }
  __syncthreads();
  for (int k = ks0; k < ks1; ++k) {
    const int cur = (k - ks0) & 1;
    const int pf = k + 2 < ks1 ? k + 2 : ks1 - 1;
    const uint8_t *xb = xs[cur];
    const u32x4 wv = *reinterpret_cast<const u32x4 *>(wp[cur] + 32 * my_row + 16 * lk);
    const float wa = wsc[cur][my_row];
    u32x4 xa[2][MI];
#pragma unroll
    for (int i = 0; i < MI; ++i)
      xa[0][i] = *reinterpret_cast<const u32x4 *>(xb + swz(32 * i + lr, 4 * lk));
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int cb = kk & 1, nb = cb ^ 1;
      if (kk < 3) {
#pragma unroll
        for (int i = 0; i < MI; ++i)
          xa[nb][i] = *reinterpret_cast<const u32x4 *>(xb + swz(32 * i + lr, 4 * lk + kk + 1));
      }
      // the 8 codes of op kk: bytes 4 kk .. 4 kk + 3 of the lane's 16
      u32x4 wop;
#pragma unroll
      for (int bb = 0; bb < 4; ++bb) {
        const float2 p = lut[(wv[kk] >> (8 * bb)) & 0xFF];
        wop[bb] = Half<AT>::pack2(p.x * wa, p.y * wa);
      }
      // staging of step k + 1 into the other buffer, one piece per op, each
      // register refilled for step k + 2 right after it was stored
      if (kk < XR) {
        store_x(cur ^ 1, kk);
        load_x(pf, kk);
      }
      if (kk == 2) {
        store_w(cur ^ 1);
        load_w(pf);
      }
#pragma unroll
      for (int i = 0; i < MI; ++i) acc[i][0] = mfma32<AT>(wop, xa[cb][i], acc[i][0]);
    }
    __syncthreads();
  }

  // LoRA bypass: acc += B (s u)^T, 16 ranks per MFMA step, first slice only
  for (int j0 = 0; j0 < (!FUSED && split == 0 ? r : 0); j0 += 16) {
    if (j0 > 0) {
      __syncthreads();
      stage_lora<BM, kSmThreads, AT>(ls_u, u, m0, M, r, j0, s, t);
      stage_lora<kSmBN, kSmThreads, AT>(ls_b, B, n0, N, r, j0, 1.0f, t);
      __syncthreads();
    }
    const u32x4 bb = lora_frag(ls_b, my_row, lk);
#pragma unroll
    for (int i = 0; i < MI; ++i) acc[i][0] = mfma32<AT>(bb, lora_frag(ls_u, 32 * i + lr, lk), acc[i][0]);
  }
  const int64_t col = n0 + 32 * wave;
  if (FUSED || nsplit > 1)
    store_tile_f32<MI, 1>(part + (int64_t)split * M * N, N, M, N, m0, col, acc, lane);
  else if (n0 + kSmBN <= N && N % 8 == 0)  // per-wave slices of 32 rows in a dead staging buffer
    store_tile_lds<AT, MI, 1>(y, N, M, m0, col, acc, &xs[0][0] + wave * 32 * (2 * 32 + 16), lane);
  else
    store_tile_t<AT, MI, 1>(y, N, M, N, m0, col, acc, lane);
}

// ===========================================================================
// Input gradient.  Contraction over the N outputs in steps of 64; the
// workgroup's output tile is 256 tokens x BX input features.  The weight
// tile (64 rows n x BX columns k) is loaded with wide coalesced reads (each
// lane takes BX/8 consecutive codes of one row), dequantised and stored in
// LDS in its natural [n][k] order; the matrix cores need 8 consecutive n of
// one column k per lane, which gfx950's transposing LDS read provides: for
// a group of 16 lanes whose 64-bit addresses name rows n0..n0+3 (lanes
// 4e..4e+3 -> row n0+e, columns c..c+15 in four 4-column pieces), output
// lane i receives column c+i of the four rows.  Two such reads give the 8
// rows of one operand.
// ===========================================================================
constexpr int kDxBC = 64;

typedef short s16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ u32x2 lds_read_tr16(const uint8_t *p) {
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4 *)(p));
  return __builtin_bit_cast(u32x2, v);
}

// Byte offset of 16-byte chunk c (8 columns) of weight-tile row n.  Chunks
// are permuted within each 256-byte bank span so that (a) the 16 lanes of a
// chunk store (two rows, eight lanes each) and (b) the 32 lanes of a
// transposing read (four rows x four chunks) touch 16 distinct bank slots.
template <int BX>
__device__ __forceinline__ int wswz(int n, int c) {
  const int p = c ^ (((n & 3) << 2) | (n & 1)) ^ (((c >> 4) & 1) << 1);
  return n * (2 * BX) + (p << 4);
}

// DROP: LoRA dropout on the bypass input; the bypass term of output (m, k)
// is multiplied by keep(m, k) / (1 - p) (dscale) before the base product is
// added to it.
// Token tile BM = 256: 8 waves as 2 (tokens) x 4 (columns), each owning a
// 128 x BX/4 block; BM = 64 (few tokens): 4 waves as 1 x 4, each owning a
// 64 x BX/4 block.
template <int BM>
struct DxShape {
  static constexpr int NT = BM == 256 ? 512 : 256;  // threads
  static constexpr int WM = BM == 256 ? 2 : 1;      // waves along tokens
  static constexpr int MI = BM / WM / 32;           // 32-row token tiles per wave
  static constexpr int XC = BM * 8 / NT;            // 16-byte dy chunks per lane per step
  static constexpr int LPR = NT / kDxBC;            // staging lanes per weight row
};

template <int BM, int BX, typename AT, typename LT, bool DQ, bool DROP>
__global__ __launch_bounds__(DxShape<BM>::NT) void k_gemm_dx(const uint16_t *__restrict__ dy, int64_t M,
                                                      const uint8_t *__restrict__ packed,
                                                      BlockScales sc, int64_t N, int64_t K,
                                                      const float *__restrict__ g,
                                                      const LT *__restrict__ A, int32_t r,
                                                      uint16_t *__restrict__ dx,
                                                      float *__restrict__ part, int nsplit,
                                                      Dropout drop, float dscale) {
  constexpr int NT = DxShape<BM>::NT, WM = DxShape<BM>::WM, MI = DxShape<BM>::MI;
  constexpr int XC = DxShape<BM>::XC, LPR = DxShape<BM>::LPR;
  constexpr int TM = 32 * MI;  // tokens per wave
  constexpr int TX = BX / 4;
  constexpr int NJ = TX / 32;
  constexpr int NU = BX / (8 * LPR);  // 32-bit code words (= 16-byte 16-bit chunks) per lane per step
  static_assert(XC == 2 || XC == 4, "dy staging is split into 2 or 4 chunks");
  static_assert(NU == 2 || NU == 4, "a lane stages 2 or 4 code words per step");
  __shared__ __attribute__((aligned(16))) uint8_t ds[2][BM * kRowBytes];  // dy [m][n], AT
  __shared__ __attribute__((aligned(16))) uint8_t wt[2][kDxBC * 2 * BX];  // W^ [n][k], AT
  __shared__ __attribute__((aligned(16))) uint8_t ls_g[BM * kLoraStride];
  __shared__ __attribute__((aligned(16))) uint8_t ls_a[BX * kLoraStride];
  __shared__ float2 lut[256];
  const int t = threadIdx.x;
  if (t < 256) lut[t] = make_float2(c_nf4[t >> 4], c_nf4[t & 15]);

  int64_t mt, kt;
  tile_of((M + BM - 1) / BM, (K + BX - 1) / BX, mt, kt);
  const int64_t m0 = mt * BM, k0 = kt * BX;
  // contraction steps of 64 outputs n; with N % 64 != 0 the last one is
  // ragged (N % 8 == 0): its dy columns past N are staged as zeros and its
  // weight rows past N repeat row N - 1 (finite values times zero)
  const int64_t NS = (N + kDxBC - 1) / kDxBC;
  // contraction slice of this workgroup (split-K: grid row blockIdx.y)
  const int split = blockIdx.y;
  const int ks0 = (int)(split * NS / nsplit), ks1 = (int)((split + 1) * NS / nsplit);

  // weight staging: lane -> row wrow of the step, 8 * NU codes from column wk
  const int wrow = t / LPR, wk = (t % LPR) * 8 * NU;
  const float mu = DQ ? sc.mu[0] : 0.0f;
  u32x4 drv[XC];
  uint32_t wr[NU];
  int wq;
  float wsig;
  // columns past K (the last column tile when K % BX != 0, K % 64 == 0)
  // load the row's last codes instead; they feed only unstored outputs
  const int64_t wcol = k0 + wk + 8 * NU <= K ? k0 + wk : K - 8 * NU;
  auto load_w = [&](int step) {
    const int64_t n = (int64_t)step * kDxBC + wrow;
    const int64_t e = (n < N ? n : N - 1) * K + wcol;
    if constexpr (NU == 2) {
      const u32x2 v = *reinterpret_cast<const u32x2 *>(packed + (e >> 1));
      wr[0] = v[0];
      wr[1] = v[1];
    } else {
      const u32x4 v = *reinterpret_cast<const u32x4 *>(packed + (e >> 1));
      wr[0] = v[0];
      wr[1] = v[1];
      wr[2] = v[2];
      wr[3] = v[3];
    }
    const int64_t b = sc.index(e >> 6);  // the lane's codes lie inside one 64-chunk
    if constexpr (DQ) {
      wq = sc.q[b];
      wsig = sc.sigma[b >> 8];
    } else {
      wq = 0;
      wsig = sc.absmax[b];
    }
  };
  // token rows past M are clamped (their outputs are never stored); a chunk
  // past N loads the row's last chunk and is staged as zeros
  const uint16_t *dy_src[XC];
#pragma unroll
  for (int i = 0; i < XC; ++i) {
    const int id = t + NT * i;
    const int64_t rr = m0 + (id >> 3) < M ? m0 + (id >> 3) : M - 1;
    dy_src[i] = dy + rr * N;
  }
  auto dy_col = [&](int step, int i) {
    return (int64_t)step * kDxBC + 8 * ((t + NT * i) & 7);
  };
  auto load_dy_chunk = [&](int step, int i) {
    const int64_t c = dy_col(step, i);
    drv[i] = *reinterpret_cast<const u32x4 *>(dy_src[i] + (c < N ? c : N - 8));
  };
  // quarter q of one step's staging: the dy chunk(s) of that quarter, and
  // the weight words assigned to it (one word = 8 codes = one 16-byte chunk)
  auto store_quarter = [&](int buf, int qq, int step) {
    if (XC == 4 || (qq & 1) == 0) {
      const int ci = XC == 4 ? qq : qq >> 1;
      const int id = t + NT * ci;
      *reinterpret_cast<u32x4 *>(ds[buf] + swz(id >> 3, id & 7)) =
          dy_col(step, ci) < N ? drv[ci] : u32x4{0u, 0u, 0u, 0u};
    }
    constexpr int every = 4 / NU;
    if (qq % every == 0) {
      const int u = qq / every;
      const float wa = DQ ? __builtin_fmaf((float)wq, wsig, mu) : wsig;
      u32x4 o;
#pragma unroll
      for (int bb = 0; bb < 4; ++bb) {
        // byte bb holds codes 2bb (high nibble) and 2bb+1 of the word
        const float2 pv = lut[(wr[u] >> (8 * bb)) & 0xFF];
        o[bb] = Half<AT>::pack2(pv.x * wa, pv.y * wa);
      }
      *reinterpret_cast<u32x4 *>(wt[buf] + wswz<BX>(wrow, (wk >> 3) + u)) = o;
    }
  };

  const int wave = t >> 6, lane = t & 63;
  const int wm = wave % WM, wn = wave / WM;
  const int lr = lane & 31, lk = lane >> 5;
  // transposing-read address of this lane within a 16-lane group:
  // row offset e = (lane & 15) / 4, column piece 4 * (lane & 3); groups
  // 1 and 3 take columns +16, groups 2 and 3 take rows +8
  const int tr_row = 8 * (lane >> 5) + ((lane & 15) >> 2);
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  auto read_b = [&](const uint8_t *wb, int kk, int j) {
    const int col = TX * wn + 32 * j + tr_col;
    const int n = 16 * kk + tr_row;
    const int off = (col & 7) * 2;
    const u32x2 lo = lds_read_tr16(wb + wswz<BX>(n, col >> 3) + off);
    const u32x2 hi = lds_read_tr16(wb + wswz<BX>(n + 4, col >> 3) + off);
    return u32x4{lo[0], lo[1], hi[0], hi[1]};
  };
  f32x16 acc[MI][NJ];
  zero_acc(&acc[0][0], MI * NJ);

  __syncthreads();  // lut
#pragma unroll
  for (int i = 0; i < XC; ++i) load_dy_chunk(ks0, i);
  load_w(ks0);
  // first 16-rank chunk of the bypass operands (g, which already holds s,
  // and A^T), used after the main loop by the first contraction slice;
  // staged here so that its loads overlap the first tile loads
  if (split == 0) {
    stage_lora<BM, NT, AT>(ls_g, g, m0, M, r, 0, 1.0f, t);
    stage_lora_t<BX, NT, AT>(ls_a, A, K, k0, r, 0, t);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) store_quarter(0, i, ks0);
#pragma unroll
  for (int i = 0; i < XC; ++i) load_dy_chunk(ks0 + 1 < ks1 ? ks0 + 1 : ks0, i);
  load_w(ks0 + 1 < ks1 ? ks0 + 1 : ks0);
  __syncthreads();
  if constexpr (DROP) {
    // LoRA bypass under dropout, first slice only, before the main loop so
    // that it needs no registers beyond the accumulator: acc = A^T g^T over
    // all ranks, then each output (m, k) is kept times 1/(1-p) or zeroed.
    // acc[i][j][v] is output row m0 + TM wm + 32 i + lr, column
    // k0 + TX wn + 32 j + 4 lk + 8 (v / 4) + v % 4; columns k .. k + 3
    // (k % 4 == 0, and K % 4 == 0) share one Philox draw.
    if (split == 0) {
      for (int j0 = 0; j0 < r; j0 += 16) {
        if (j0 > 0) {
          __syncthreads();
          stage_lora<BM, NT, AT>(ls_g, g, m0, M, r, j0, 1.0f, t);
          stage_lora_t<BX, NT, AT>(ls_a, A, K, k0, r, j0, t);
          __syncthreads();
        }
        u32x4 ga[MI], ab[NJ];
#pragma unroll
        for (int i = 0; i < MI; ++i) ga[i] = lora_frag(ls_g, TM * wm + 32 * i + lr, lk);
#pragma unroll
        for (int j = 0; j < NJ; ++j) ab[j] = lora_frag(ls_a, TX * wn + 32 * j + lr, lk);
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
          for (int j = 0; j < NJ; ++j) acc[i][j] = mfma32<AT>(ab[j], ga[i], acc[i][j]);
      }
#pragma unroll
      for (int i = 0; i < MI; ++i) {
        const uint64_t m = (uint64_t)(m0 + TM * wm + 32 * i + lr);
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
          for (int qq = 0; qq < 4; ++qq) {
            const int64_t k = k0 + TX * wn + 32 * j + 8 * qq + 4 * lk;
            const uint32_t bits = dropout_keep4(drop, m * (uint64_t)K + (uint64_t)k);
#pragma unroll
            for (int e = 0; e < 4; ++e)
              acc[i][j][4 * qq + e] = (bits >> e) & 1u ? dscale * acc[i][j][4 * qq + e] : 0.0f;
          }
      }
    }
  }
  for (int k = ks0; k < ks1; ++k) {
    const int cur = (k - ks0) & 1;
    const int pf = k + 2 < ks1 ? k + 2 : ks1 - 1;
    const uint8_t *db = ds[cur];
    const uint8_t *wb = wt[cur];
    u32x4 a[2][MI], b[2][NJ];
#pragma unroll
    for (int i = 0; i < MI; ++i)
      a[0][i] = *reinterpret_cast<const u32x4 *>(db + swz(TM * wm + 32 * i + lr, lk));
#pragma unroll
    for (int j = 0; j < NJ; ++j) b[0][j] = read_b(wb, 0, j);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int cb = kk & 1, nb = cb ^ 1;
      if (kk < 3) {
        const int chunk = 2 * (kk + 1) + lk;
#pragma unroll
        for (int i = 0; i < MI; ++i)
          a[nb][i] = *reinterpret_cast<const u32x4 *>(db + swz(TM * wm + 32 * i + lr, chunk));
#pragma unroll
        for (int j = 0; j < NJ; ++j) b[nb][j] = read_b(wb, kk + 1, j);
      }
      // each dy chunk is reloaded right after it was stored
      store_quarter(cur ^ 1, kk, k + 1 < ks1 ? k + 1 : ks1 - 1);
      if (XC == 4) load_dy_chunk(pf, kk);
      else if ((kk & 1) == 0) load_dy_chunk(pf, kk >> 1);
      if (kk == 3) load_w(pf);
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j) acc[i][j] = mfma32<AT>(b[cb][j], a[cb][i], acc[i][j]);
    }
    __syncthreads();
  }

  // LoRA bypass: acc += A^T g^T, 16 ranks per MFMA step (first slice only;
  // with dropout it ran before the main loop)
  for (int j0 = 0; j0 < (split == 0 && !DROP ? r : 0); j0 += 16) {
    if (j0 > 0) {
      __syncthreads();
      stage_lora<BM, NT, AT>(ls_g, g, m0, M, r, j0, 1.0f, t);
      stage_lora_t<BX, NT, AT>(ls_a, A, K, k0, r, j0, t);
      __syncthreads();
    }
    u32x4 ga[MI], ab[NJ];
#pragma unroll
    for (int i = 0; i < MI; ++i) ga[i] = lora_frag(ls_g, TM * wm + 32 * i + lr, lk);
#pragma unroll
    for (int j = 0; j < NJ; ++j) ab[j] = lora_frag(ls_a, TX * wn + 32 * j + lr, lk);
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j) acc[i][j] = mfma32<AT>(ab[j], ga[i], acc[i][j]);
  }
  if (nsplit > 1)
    store_tile_f32<MI, NJ>(part + (int64_t)split * M * K, K, M, K, m0 + TM * wm, k0 + TX * wn,
                           acc, lane);
  else if (k0 + BX <= K)  // per-wave slices of 32 rows in a dead staging buffer
    store_tile_lds<AT, MI, NJ>(dx, K, M, m0 + TM * wm, k0 + TX * wn, acc,
                           (BM == 256 ? &ds[0][0] : &wt[0][0]) + wave * 32 * (2 * TX + 16), lane);
  else  // the ragged last column tile (K % BX != 0)
    store_tile_t<AT, MI, NJ>(dx, K, M, K, m0 + TM * wm, k0 + TX * wn, acc, lane);
}

// Split-K: a launch with fewer tiles than the chip runs at once (a few
// token tiles) leaves units idle while each workgroup walks the whole
// contraction.  Its contraction is then split into S slices (grid rows) that
// write fp32 partial tiles, summed in fixed order by k_reduce_split.  For the
// few-token kernels S minimises (waves of `slots` workgroups: 512 for them,
// as they run up to four per unit but gain little past two) x (steps per
// slice + ~4 steps of prologue and epilogue), keeps >= 8 steps per slice and
// the partial buffer <= 64 MB, and prefers the smaller S on ties; it
// depends only on the shape.
static int split_count(int64_t tiles, int64_t steps, int64_t M, int64_t cols, int64_t slots,
                       int64_t scap = 16, int64_t cap = (int64_t)64 << 20) {
  if (tiles >= slots || tiles <= 0 || cols % 4 != 0) return 1;
  int64_t smax = steps / 8;
  if (smax > scap) smax = scap;
  const int64_t per = M * cols * 4;
  if (per > 0 && smax > cap / per) smax = cap / per;
  int best = 1;
  double best_cost = (double)steps + 4.0;  // S = 1: one wave
  for (int64_t S = 2; S <= smax; ++S) {
    const double waves = (double)((tiles * S + slots - 1) / slots);
    const double cost = waves * ((double)steps / (double)S + 4.0);
    if (cost < best_cost) {
      best_cost = cost;
      best = (int)S;
    }
  }
  return best;
}

// Plan of a 256-token launch: output tile width bn (256, or 128) and
// split-K count S, from a cost model in units of one contraction step of a
// 256 x 256 tile:
//     waves(tiles(bn) S / 256) (steps / S  c(bn) + 4)
//   + [S > 1] 8 M cols S / kPartialBytesPerStep
// c(256) = 1 and c(128) = 0.62 are the measured per-step times of the two
// tiles relative to each other (1.9 and 1.2 us on the 8B MLP shapes: the
// wider tile does twice the work per step for 1.6x the time); the second
// term is the fp32 partial tiles of a split launch, written and read back
// (8 bytes per output per slice), at ~7.7 MB per step unit (~4 TB/s over a
// 1.9 us step).  Slices keep >= 8 steps each and the partial buffer stays
// <= 256 MB.  The smallest cost wins; ties go to the wider tile and the
// smaller S.  It depends only on the shape (and on whether splitting is
// allowed), so the workspace query and the launch agree.
struct TilePlan {
  int bn, S;
};
constexpr double kPartialBytesPerStep = 7.7e6;

static TilePlan plan_tiles(int64_t M, int64_t cols, int64_t steps, bool wide_ok, bool split_ok) {
  const int64_t mt = (M + kBM - 1) / kBM;
  TilePlan best{128, 1};
  double best_cost = 1e300;
  for (int bn = 256; bn >= 128; bn -= 128) {
    if (bn == 256 && !wide_ok) continue;
    const double c = bn == 256 ? 1.0 : 0.62;
    const int64_t tiles = mt * ((cols + bn - 1) / bn);
    int64_t smax = (split_ok && cols % 4 == 0) ? steps / 8 : 1;
    if (smax > 16) smax = 16;
    const int64_t per = M * cols * 4;
    const int64_t cap = (int64_t)256 << 20;
    if (per > 0 && smax > cap / per) smax = cap / per;
    if (smax < 1) smax = 1;
    for (int64_t S = 1; S <= smax; ++S) {
      const double waves = (double)((tiles * S + 255) / 256);
      double cost = waves * ((double)steps / (double)S * c + 4.0);
      if (S > 1) cost += 8.0 * (double)M * (double)cols * (double)S / kPartialBytesPerStep;
      if (cost < best_cost * (1.0 - 1e-9)) {
        best_cost = cost;
        best = TilePlan{bn, (int)S};
      }
    }
  }
  return best;
}

// Forward tile (k_gemm_fwd_small): 64 tokens x 128 outputs up to 64 tokens,
// 128 tokens x 128 outputs up to kFwdMidM tokens, else 256 tokens x the
// planned width (k_gemm_fwd).  Measured on the 8B MLP's gate and down shapes
// at 80-512 tokens: from 65 to 128 tokens the 128-token tile is 10-13 %
// faster than two 64-token tiles; from 160 on it ties with the 256-token
// tile or loses.
constexpr int64_t kFwdMidM = 128;

static int fwd_small_bm(int64_t M) { return M <= kSmBM ? 64 : (M <= kFwdMidM ? 128 : 0); }

// With 64-token tiles and a long contraction (>= 128 steps) the split model
// counts the kernel's real residency (four workgroups per unit, 1024 slots)
// and allows up to 32 slices: measured on the 8B MLP's down shape
// (4096x14336, 224 steps) the forward at 17 / 64 tokens runs 18 / 10 % faster
// (28.9 -> 23.7, 34.7 -> 31.4 us); on the gate shape (64 steps) the same
// model is 3-7 % slower, so shorter contractions keep 512 slots and 16.  Its
// partials stay within 28 MiB, so that every forward of up to 96 tokens on
// these shapes still fits the allocation-free entry point's 32 MiB.
static int fwd_split(int64_t M, int64_t N, int64_t K) {
  const int64_t bm = fwd_small_bm(M);
  const bool deep = bm == 64 && (K >> 6) >= 128;
  if (bm)
    return split_count(((M + bm - 1) / bm) * ((N + kSmBN - 1) / kSmBN), K >> 6, M, N,
                       deep ? 1024 : 512, deep ? 32 : 16,
                       deep ? (int64_t)28 << 20 : (int64_t)64 << 20);
  return plan_tiles(M, N, K >> 6, true, true).S;
}

// Input-gradient tile: 64 tokens x 128 columns up to 64 tokens, 128 x 128 up
// to kDxMidM tokens, else 256 tokens x the planned width (256 needs K % 256
// == 0).  The same measurement as the forward's: the 128-token tile is 10-14
// % faster from 65 to 128 tokens and 6-8 % slower from 160 on.
constexpr int64_t kDxMidM = 128;

static int dx_small_bm(int64_t M) { return M <= 64 ? 64 : (M <= kDxMidM ? 128 : 0); }

static int dx_split(int64_t M, int64_t N, int64_t K) {
  const int64_t steps = (N + kDxBC - 1) / kDxBC;
  const int64_t bm = dx_small_bm(M);
  if (bm) return split_count(((M + bm - 1) / bm) * ((K + 127) / 128), steps, M, K, 512);
  return plan_tiles(M, K, steps, K % 256 == 0, true).S;
}

size_t gemm_fwd_partial_floats(int64_t M, int64_t N, int64_t K) {
  const int S = fwd_split(M, N, K);
  return S > 1 ? (size_t)S * (size_t)M * (size_t)N : 0;
}

size_t gemm_dx_partial_floats(int64_t M, int64_t N, int64_t K) {
  const int S = dx_split(M, N, K);
  return S > 1 ? (size_t)S * (size_t)M * (size_t)K : 0;
}

static int reduce_split(int act_dtype, const float *part, int S, int64_t count, uint16_t *out,
                        hipStream_t stream) {
  const int64_t n4 = count / 4;
  with_half(act_dtype, [&](auto *tag) {
    hipLaunchKernelGGL((k_reduce_split<elem_of<decltype(tag)>>), dim3((unsigned)((n4 + 255) / 256)),
                       dim3(256), 0, stream, part, S, count, out);
  });
  QL_HIP_CHECK_LAUNCH();
  return QL_OK;
}

// A 16-bit LoRA factor has the activations' format (checked by the caller):
// LT is float or AT.
int launch_gemm_fwd(const void *xv, int act_dtype, int64_t M, const uint8_t *packed,
                    BlockScales sc, int64_t N, int64_t K, const float *u, const void *B,
                    int lora_dtype, int32_t r, float s, void *yv, hipStream_t stream,
                    float *part) {
  const uint16_t *x = (const uint16_t *)xv;
  uint16_t *y = (uint16_t *)yv;
  const bool dq = sc.absmax == nullptr;
  if (const int bm = fwd_small_bm(M)) {
    const int64_t G = ((M + bm - 1) / bm) * ((N + kSmBN - 1) / kSmBN);
    const int S = part ? fwd_split(M, N, K) : 1;
#define QL_FWS(BMV, LT, DQV)                                                                     \
  hipLaunchKernelGGL((k_gemm_fwd_small<BMV, AT, LT, DQV, false>), dim3((unsigned)G, (unsigned)S), \
                     dim3(kSmThreads), 0, stream, x, M, packed, sc, N, K, u, (const LT *)B, r, s, \
                     y, part, S, (const LT *)nullptr, (float *)nullptr, 0, 0, Dropout{0u, 0u, 0u})
#define QL_FWS_BM(LT, DQV) \
  do { if (bm == 64) QL_FWS(64, LT, DQV); else QL_FWS(128, LT, DQV); } while (0)
    with_half(act_dtype, [&](auto *tag) {
      using AT = elem_of<decltype(tag)>;
      if (lora_dtype == QL_F32) {
        if (dq) QL_FWS_BM(float, true); else QL_FWS_BM(float, false);
      } else {
        if (dq) QL_FWS_BM(AT, true); else QL_FWS_BM(AT, false);
      }
    });
#undef QL_FWS_BM
#undef QL_FWS
    QL_HIP_CHECK_LAUNCH();
    if (S > 1) return reduce_split(act_dtype, part, S, M * N, y, stream);
    return QL_OK;
  }
  const TilePlan pl = plan_tiles(M, N, K >> 6, true, part != nullptr);
  const int bn = pl.bn, S = pl.S;
  const int64_t G = ((M + kBM - 1) / kBM) * ((N + bn - 1) / bn);
#define QL_FWD(BNV, LT, DQV)                                                                     \
  hipLaunchKernelGGL((k_gemm_fwd<BNV, AT, LT, DQV>), dim3((unsigned)G, (unsigned)S),            \
                     dim3(kThreads), 0, stream, x, M, packed, sc, N, K, u, (const LT *)B, r, s,  \
                     y, part, S)
#define QL_FWD_DQ(BNV, LT) \
  do { if (dq) QL_FWD(BNV, LT, true); else QL_FWD(BNV, LT, false); } while (0)
  with_half(act_dtype, [&](auto *tag) {
    using AT = elem_of<decltype(tag)>;
    if (bn == 256) {
      if (lora_dtype == QL_F32) QL_FWD_DQ(256, float);
      else QL_FWD_DQ(256, AT);
    } else {
      if (lora_dtype == QL_F32) QL_FWD_DQ(128, float);
      else QL_FWD_DQ(128, AT);
    }
  });
#undef QL_FWD_DQ
#undef QL_FWD
  QL_HIP_CHECK_LAUNCH();
  if (S > 1) return reduce_split(act_dtype, part, S, M * N, y, stream);
  return QL_OK;
}

// Up to 128 tokens (the few-token tiles) the u slices and the slice sum with
// the bypass (two launches) beat u in launches of its own plus a split-K sum:
// measured at 65-128 tokens with 128-token tiles, the fused form is 10-16 %
// faster on the 8B MLP's down shape (4096x14336, the long contraction whose
// u costs most) and within 2 % either way on the gate shape (14336x4096).
constexpr int64_t kFusedMaxM = 128;
bool gemm_fwd_fused_preferred(int64_t M) { return M > 16 && M <= kFusedMaxM; }

size_t gemm_fwd_fused_partial_floats(int64_t M, int64_t N, int64_t K, int32_t r) {
  if (!gemm_fwd_fused_preferred(M)) return 0;
  return (size_t)fwd_split(M, N, K) * M * N + (size_t)u_slices(K).U * M * r;
}

int launch_gemm_fwd_fused(const void *xv, int act_dtype, int64_t M, const uint8_t *packed,
                          BlockScales sc, int64_t N, int64_t K, const void *A, const void *B,
                          int lora_dtype, int32_t r, float s, void *y, float *u_save,
                          hipStream_t stream, float *part, const Dropout *drop, float dscale) {
  const uint16_t *x = (const uint16_t *)xv;
  const Dropout dr = drop ? *drop : Dropout{0u, 0u, 0u};
  const bool dq = sc.absmax == nullptr;
  const int bm = fwd_small_bm(M);
  const int64_t G = ((M + bm - 1) / bm) * ((N + kSmBN - 1) / kSmBN);
  const int S = fwd_split(M, N, K);
  const USlices us = u_slices(K);
  const int MT = (int)((M + 15) / 16), JT = (r + 15) / 16;
  float *upart = part + (size_t)S * M * N;
  const dim3 grid((unsigned)(G + (int64_t)us.U * JT * MT), (unsigned)S);
#define QL_FWF(BMV, LT, DQV)                                                                     \
  hipLaunchKernelGGL((k_gemm_fwd_small<BMV, AT, LT, DQV, true>), grid, dim3(kSmThreads), 0, stream, \
                     x, M, packed, sc, N, K, (const float *)nullptr, (const LT *)B, r, s,         \
                     (uint16_t *)nullptr, part, S, (const LT *)A, upart, us.uc, MT, dr)
#define QL_FWF_BM(LT, DQV) \
  do { if (bm == 64) QL_FWF(64, LT, DQV); else QL_FWF(128, LT, DQV); } while (0)
  with_half(act_dtype, [&](auto *tag) {
    using AT = elem_of<decltype(tag)>;
    if (lora_dtype == QL_F32) {
      if (dq) QL_FWF_BM(float, true); else QL_FWF_BM(float, false);
    } else {
      if (dq) QL_FWF_BM(AT, true); else QL_FWF_BM(AT, false);
    }
  });
#undef QL_FWF_BM
#undef QL_FWF
  QL_HIP_CHECK_LAUNCH();
  return launch_fwd_finish(act_dtype, lora_dtype, part, S, upart, us.U, M, N, r, B, s, y, u_save,
                           stream, drop ? dscale : 1.0f);
}

// 16-byte loads of dy rows and of 8-code words: N % 8 == 0 and K % 64 == 0
bool gemm_dx_supported(int64_t N, int64_t K) { return N % 8 == 0 && N >= 8 && K % 64 == 0; }

int launch_gemm_dx(const void *dyv, int act_dtype, int64_t M, const uint8_t *packed,
                   BlockScales sc, int64_t N, int64_t K, const float *g, const void *A,
                   int lora_dtype, int32_t r, void *dxv, hipStream_t stream, float *part,
                   const Dropout *drop, float drop_scale) {
  const uint16_t *dy = (const uint16_t *)dyv;
  uint16_t *dx = (uint16_t *)dxv;
  const Dropout dr = drop ? *drop : Dropout{0u, 0u, 0u};
  const int sbm = dx_small_bm(M);
  const int bm = sbm ? sbm : kBM;
  const TilePlan pl = sbm ? TilePlan{128, part ? dx_split(M, N, K) : 1}
                          : plan_tiles(M, K, (N + kDxBC - 1) / kDxBC, K % 256 == 0,
                                       part != nullptr);
  const int bx = pl.bn, S = pl.S;
  const int64_t G = ((M + bm - 1) / bm) * ((K + bx - 1) / bx);
  const bool dq = sc.absmax == nullptr;
#define QL_DX(BMV, BXV, LT, DQV, DRV)                                                            \
  hipLaunchKernelGGL((k_gemm_dx<BMV, BXV, AT, LT, DQV, DRV>), dim3((unsigned)G, (unsigned)S),   \
                     dim3(DxShape<BMV>::NT), 0, stream, dy, M, packed, sc, N, K, g, (const LT *)A, \
                     r, dx, part, S, dr, drop_scale)
#define QL_DX_DR(BMV, BXV, LT, DQV) \
  do { if (drop) QL_DX(BMV, BXV, LT, DQV, true); else QL_DX(BMV, BXV, LT, DQV, false); } while (0)
#define QL_DX_DQ(BMV, BXV, LT) \
  do { if (dq) QL_DX_DR(BMV, BXV, LT, true); else QL_DX_DR(BMV, BXV, LT, false); } while (0)
#define QL_DX_LT(BMV, BXV) \
  do { if (lora_dtype == QL_F32) QL_DX_DQ(BMV, BXV, float); else QL_DX_DQ(BMV, BXV, AT); } while (0)
  with_half(act_dtype, [&](auto *tag) {
    using AT = elem_of<decltype(tag)>;
    if (sbm == 64) QL_DX_LT(64, 128);
    else if (sbm == 128) QL_DX_LT(128, 128);
    else if (bx == 256) QL_DX_LT(256, 256);
    else QL_DX_LT(256, 128);
  });
#undef QL_DX_LT
#undef QL_DX_DQ
#undef QL_DX_DR
#undef QL_DX
  QL_HIP_CHECK_LAUNCH();
  if (S > 1) return reduce_split(act_dtype, part, S, M * K, dx, stream);
  return QL_OK;
}

}  // namespace qlora
