// gemm.hip -- matrix-core (bf16 MFMA, fp32 accumulate) products of the QLoRA
// layer for many tokens:
//
//   forward:        y  = x W^^T + s u B^T   (26. QLoRA and 4bit Quantization, Step 3)
//   input gradient: dx = dy W^  + g A       (22. QLoRA and 4bit Quantization, Step 1:
//                                            the gradient flows through the frozen base)
//
// W^ is never materialised: each workgroup dequantises the NF4 tile it needs
// (26. ..., Step 4: table[index] * scale; 22. ..., Step 3: restored to a 16-bit
// float for the product) straight into LDS as bf16 and feeds the matrix
// cores from there.  The rank-r bypass is folded into the same accumulators
// as extra 16-deep MFMA steps (u and g are fp32 in memory and are rounded to
// bf16 for those steps).
//
// Tiles: 256 (tokens) x 128 (outputs) per workgroup, contraction step 64
// (= one NF4 block of every weight row in the forward), 8 waves of 64 x 64.
// LDS rows are 64 bf16 = 8 chunks of 16 bytes; chunk c of row r is stored at
// position c ^ (r & 7) so that 8 consecutive rows read at the same logical
// chunk hit 8 different bank groups.
//
// v_mfma_f32_32x32x16_bf16 layout (gfx950): A lane l holds A[l % 32][8*(l/32)
// .. +8], B lane l holds B[8*(l/32) .. +8][l % 32], result register v of lane
// l is D[8*(v/4) + 4*(l/32) + v%4][l % 32].
#include "kernels.h"

namespace qlora {

constexpr int kBM = 256;
constexpr int kBN = 128;
constexpr int kBK = 64;
constexpr int kThreads = 512;

__device__ __forceinline__ int swz(int row, int chunk) { return row * 128 + ((chunk ^ (row & 7)) << 4); }

__device__ __forceinline__ f32x16 mfma32(const u32x4 &a, const u32x4 &b, const f32x16 &c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Workgroup -> tile.  Consecutive workgroup ids are spread round-robin over
// the 8 XCDs; remap so that each XCD receives a contiguous range of logical
// tiles, ordered output-column fastest: an XCD then keeps the same token tile
// (activations) in its L2 while it walks across the weight.
__device__ __forceinline__ void tile_of(int64_t mt_count, int64_t nt_count, int64_t &mt, int64_t &nt) {
  const int64_t G = mt_count * nt_count;
  int64_t bid = blockIdx.x;
  int64_t L = (G % 8 == 0) ? (bid % 8) * (G / 8) + bid / 8 : bid;
  mt = L / nt_count;
  nt = L % nt_count;
}

template <typename T>
__device__ __forceinline__ void load8_as_bf16(const T *p, int64_t i, bool ok, u32x4 &out);
template <>
__device__ __forceinline__ void load8_as_bf16<uint16_t>(const uint16_t *p, int64_t i, bool ok,
                                                        u32x4 &out) {
  if (ok) {
    out = *reinterpret_cast<const u32x4 *>(p + i);
  } else {
    out = u32x4{0u, 0u, 0u, 0u};
  }
}
template <>
__device__ __forceinline__ void load8_as_bf16<float>(const float *p, int64_t i, bool ok, u32x4 &out) {
  if (ok) {
    const float4 a = *reinterpret_cast<const float4 *>(p + i);
    const float4 b = *reinterpret_cast<const float4 *>(p + i + 4);
    out = u32x4{pack_bf16x2(a.x, a.y), pack_bf16x2(a.z, a.w), pack_bf16x2(b.x, b.y),
                pack_bf16x2(b.z, b.w)};
  } else {
    out = u32x4{0u, 0u, 0u, 0u};
  }
}

// Eight consecutive entries j0..j0+7 of a length-r row (zero past r), as bf16.
template <typename T>
__device__ __forceinline__ u32x4 lora_row8(const T *row, int j0, int r, float scale) {
  float v[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = (j0 + e < r) ? scale * load_as_f32(row, j0 + e) : 0.0f;
  return u32x4{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
               pack_bf16x2(v[6], v[7])};
}

// ===========================================================================
// Forward
// ===========================================================================
template <typename LT>
__global__ __launch_bounds__(kThreads) void k_gemm_fwd(const uint16_t *__restrict__ x, int64_t M,
                                                       const uint8_t *__restrict__ packed,
                                                       BlockScales sc, int64_t N, int64_t K,
                                                       const float *__restrict__ u,
                                                       const LT *__restrict__ B, int32_t r,
                                                       float s, uint16_t *__restrict__ y) {
  __shared__ __attribute__((aligned(16))) uint8_t xs[kBM * 128];
  __shared__ __attribute__((aligned(16))) uint8_t ws[kBN * 128];
  __shared__ float2 lut[256];
  const int t = threadIdx.x;
  if (t < 256) lut[t] = make_float2(c_nf4[t >> 4], c_nf4[t & 15]);

  int64_t mt, nt;
  tile_of((M + kBM - 1) / kBM, (N + kBN - 1) / kBN, mt, nt);
  const int64_t m0 = mt * kBM, n0 = nt * kBN;
  const int64_t KB = K >> 6;

  // global -> register staging
  u32x4 xr[4];
  u32x2 wr;
  float wa;
  const int w_row = t >> 2, w_part = t & 3;
  const int64_t w_n = n0 + w_row;
  const bool w_ok = w_n < N;

  auto load_stage = [&](int64_t k0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int id = t + kThreads * i;
      const int row = id >> 3, c = id & 7;
      const int64_t m = m0 + row;
      load8_as_bf16<uint16_t>(x, m * K + k0 + 8 * c, m < M, xr[i]);
    }
    if (w_ok) {
      wr = *reinterpret_cast<const u32x2 *>(packed + ((w_n * K + k0) >> 1) + 8 * w_part);
      wa = sc(w_n * KB + (k0 >> 6));
    } else {
      wr = u32x2{0u, 0u};
      wa = 0.0f;
    }
  };
  auto store_stage = [&]() {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int id = t + kThreads * i;
      const int row = id >> 3, c = id & 7;
      *reinterpret_cast<u32x4 *>(xs + swz(row, c)) = xr[i];
    }
    uint32_t d[8];
#pragma unroll
    for (int bi = 0; bi < 8; ++bi) {
      const uint32_t word = bi < 4 ? wr.x : wr.y;
      const float2 p = lut[(word >> (8 * (bi & 3))) & 0xFF];
      d[bi] = pack_bf16x2(p.x * wa, p.y * wa);
    }
    *reinterpret_cast<u32x4 *>(ws + swz(w_row, 2 * w_part)) = u32x4{d[0], d[1], d[2], d[3]};
    *reinterpret_cast<u32x4 *>(ws + swz(w_row, 2 * w_part + 1)) = u32x4{d[4], d[5], d[6], d[7]};
  };

  const int wave = t >> 6, lane = t & 63;
  const int wm = wave & 3, wn = wave >> 2;
  const int lr = lane & 31, lk = lane >> 5;
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  __syncthreads();  // lut
  load_stage(0);
  for (int64_t k0 = 0; k0 < K; k0 += kBK) {
    store_stage();
    __syncthreads();
    if (k0 + kBK < K) load_stage(k0 + kBK);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int chunk = 2 * kk + lk;
      u32x4 a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        a[i] = *reinterpret_cast<const u32x4 *>(xs + swz(64 * wm + 32 * i + lr, chunk));
#pragma unroll
      for (int j = 0; j < 2; ++j)
        b[j] = *reinterpret_cast<const u32x4 *>(ws + swz(64 * wn + 32 * j + lr, chunk));
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma32(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }

  // LoRA bypass: acc += (s u) B^T, 16 ranks per MFMA step.
  for (int j0 = 0; j0 < r; j0 += 16) {
    u32x4 a[2], b[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int64_t m = m0 + 64 * wm + 32 * i + lr;
      a[i] = (m < M) ? lora_row8(u + m * r, j0 + 8 * lk, r, s) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t n = n0 + 64 * wn + 32 * j + lr;
      b[j] = (n < N) ? lora_row8(B + n * r, j0 + 8 * lk, r, 1.0f) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[i][j] = mfma32(a[i], b[j], acc[i][j]);
  }

#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t n = n0 + 64 * wn + 32 * j + lr;
      if (n >= N) continue;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t m = m0 + 64 * wm + 32 * i + 8 * (v >> 2) + 4 * lk + (v & 3);
        if (m < M) y[m * N + n] = f32_to_bf16_bits(acc[i][j][v]);
      }
    }
}

// ===========================================================================
// Input gradient.  Contraction over the N outputs in steps of 64; the
// workgroup's output tile is 256 tokens x 128 input features.  The weight
// tile (64 rows n x 128 columns k, two NF4 blocks per row) is staged raw in
// LDS, then every lane dequantises a 2 (n) x 8 (k) patch and writes it
// transposed ([k][n], n contiguous) so the matrix cores read 8 consecutive n
// per lane.
// ===========================================================================
constexpr int kDxBX = 128;
constexpr int kDxBC = 64;

template <typename LT>
__global__ __launch_bounds__(kThreads) void k_gemm_dx(const uint16_t *__restrict__ dy, int64_t M,
                                                      const uint8_t *__restrict__ packed,
                                                      BlockScales sc, int64_t N, int64_t K,
                                                      const float *__restrict__ g,
                                                      const LT *__restrict__ A, int32_t r,
                                                      uint16_t *__restrict__ dx) {
  __shared__ __attribute__((aligned(16))) uint8_t ds[kBM * 128];      // [m][n] bf16
  __shared__ __attribute__((aligned(16))) uint8_t wt[kDxBX * 128];    // [k][n] bf16
  __shared__ __attribute__((aligned(16))) uint8_t wraw[kDxBC * 64];   // [n][64 bytes]
  __shared__ float2 lut[256];
  const int t = threadIdx.x;
  if (t < 256) lut[t] = make_float2(c_nf4[t >> 4], c_nf4[t & 15]);

  int64_t mt, kt;
  tile_of((M + kBM - 1) / kBM, K / kDxBX, mt, kt);
  const int64_t m0 = mt * kBM, k0 = kt * kDxBX;
  const int64_t KB = K >> 6;

  u32x4 dr[4];
  u32x2 wr;
  float wa0, wa1;
  const int raw_row = t >> 3, raw_part = t & 7;  // staging of the packed tile
  const int pp = t & 31, kg = t >> 5;            // transposing dequant: rows 2pp, 2pp+1; k 8kg..+8

  auto load_stage = [&](int64_t n0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int id = t + kThreads * i;
      const int row = id >> 3, c = id & 7;
      const int64_t m = m0 + row;
      load8_as_bf16<uint16_t>(dy, m * N + n0 + 8 * c, m < M, dr[i]);
    }
    const int64_t n = n0 + raw_row;
    wr = *reinterpret_cast<const u32x2 *>(packed + ((n * K + k0) >> 1) + 8 * raw_part);
    const int64_t blk = (k0 >> 6) + (kg >> 3);
    wa0 = sc((n0 + 2 * pp) * KB + blk);
    wa1 = sc((n0 + 2 * pp + 1) * KB + blk);
  };

  const int wave = t >> 6, lane = t & 63;
  const int wm = wave & 3, wn = wave >> 2;
  const int lr = lane & 31, lk = lane >> 5;
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  __syncthreads();  // lut
  load_stage(0);
  for (int64_t n0 = 0; n0 < N; n0 += kDxBC) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int id = t + kThreads * i;
      *reinterpret_cast<u32x4 *>(ds + swz(id >> 3, id & 7)) = dr[i];
    }
    *reinterpret_cast<u32x2 *>(wraw + raw_row * 64 + 8 * raw_part) = wr;
    __syncthreads();
    {
      // rows 2pp and 2pp+1, columns 8kg..8kg+7 (4 bytes of each row)
      const uint32_t w0 = *reinterpret_cast<const uint32_t *>(wraw + (2 * pp) * 64 + 4 * kg);
      const uint32_t w1 = *reinterpret_cast<const uint32_t *>(wraw + (2 * pp + 1) * 64 + 4 * kg);
#pragma unroll
      for (int bi = 0; bi < 4; ++bi) {
        const float2 p0 = lut[(w0 >> (8 * bi)) & 0xFF];
        const float2 p1 = lut[(w1 >> (8 * bi)) & 0xFF];
        const int kr = 8 * kg + 2 * bi;
        const int off = ((pp >> 2) ^ (kr & 7)) * 16 + (pp & 3) * 4;
        const int off1 = ((pp >> 2) ^ ((kr + 1) & 7)) * 16 + (pp & 3) * 4;
        *reinterpret_cast<uint32_t *>(wt + kr * 128 + off) = pack_bf16x2(p0.x * wa0, p1.x * wa1);
        *reinterpret_cast<uint32_t *>(wt + (kr + 1) * 128 + off1) =
            pack_bf16x2(p0.y * wa0, p1.y * wa1);
      }
    }
    __syncthreads();
    if (n0 + kDxBC < N) load_stage(n0 + kDxBC);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int chunk = 2 * kk + lk;
      u32x4 a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        a[i] = *reinterpret_cast<const u32x4 *>(ds + swz(64 * wm + 32 * i + lr, chunk));
#pragma unroll
      for (int j = 0; j < 2; ++j)
        b[j] = *reinterpret_cast<const u32x4 *>(wt + swz(64 * wn + 32 * j + lr, chunk));
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma32(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }

  // LoRA bypass: acc += g A, 16 ranks per MFMA step (g already holds s).
  for (int j0 = 0; j0 < r; j0 += 16) {
    u32x4 a[2], b[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int64_t m = m0 + 64 * wm + 32 * i + lr;
      a[i] = (m < M) ? lora_row8(g + m * r, j0 + 8 * lk, r, 1.0f) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t k = k0 + 64 * wn + 32 * j + lr;
      float v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int jj = j0 + 8 * lk + e;
        v[e] = (jj < r) ? load_as_f32(A, (int64_t)jj * K + k) : 0.0f;
      }
      b[j] = u32x4{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                   pack_bf16x2(v[6], v[7])};
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[i][j] = mfma32(a[i], b[j], acc[i][j]);
  }

#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t k = k0 + 64 * wn + 32 * j + lr;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t m = m0 + 64 * wm + 32 * i + 8 * (v >> 2) + 4 * lk + (v & 3);
        if (m < M) dx[m * K + k] = f32_to_bf16_bits(acc[i][j][v]);
      }
    }
}

int launch_gemm_fwd(const uint16_t *x, int64_t M, const uint8_t *packed, BlockScales sc,
                    int64_t N, int64_t K, const float *u, const void *B, int lora_dtype, int32_t r,
                    float s, uint16_t *y, hipStream_t stream) {
  const int64_t G = ((M + kBM - 1) / kBM) * ((N + kBN - 1) / kBN);
  if (lora_dtype == QL_BF16)
    hipLaunchKernelGGL(k_gemm_fwd<uint16_t>, dim3((unsigned)G), dim3(kThreads), 0, stream, x, M,
                       packed, sc, N, K, u, (const uint16_t *)B, r, s, y);
  else
    hipLaunchKernelGGL(k_gemm_fwd<float>, dim3((unsigned)G), dim3(kThreads), 0, stream, x, M,
                       packed, sc, N, K, u, (const float *)B, r, s, y);
  QL_HIP_CHECK_LAUNCH();
  return QL_OK;
}

int launch_gemm_dx(const uint16_t *dy, int64_t M, const uint8_t *packed, BlockScales sc,
                   int64_t N, int64_t K, const float *g, const void *A, int lora_dtype, int32_t r,
                   uint16_t *dx, hipStream_t stream) {
  const int64_t G = ((M + kBM - 1) / kBM) * (K / kDxBX);
  if (lora_dtype == QL_BF16)
    hipLaunchKernelGGL(k_gemm_dx<uint16_t>, dim3((unsigned)G), dim3(kThreads), 0, stream, dy, M,
                       packed, sc, N, K, g, (const uint16_t *)A, r, dx);
  else
    hipLaunchKernelGGL(k_gemm_dx<float>, dim3((unsigned)G), dim3(kThreads), 0, stream, dy, M,
                       packed, sc, N, K, g, (const float *)A, r, dx);
  QL_HIP_CHECK_LAUNCH();
  return QL_OK;
}

}  // namespace qlora
