// gemv.hip -- decode-sized forward of the QLoRA layer (M <= 16 tokens, bf16),
// one kernel launch per call:
//
//   u = x A^T,   y = x W^^T + s u B^T     (26. QLoRA and 4bit Quantization, Step 3)
//
// Memory-bound: the packed 4-bit weight is the dominant traffic.  Each
// workgroup owns 16 weight rows; its 8 waves split the K dimension.  A lane
// of a wave holds 16 consecutive indices (8 bytes) of one row per NF4 block,
// so one block of one row is read by 4 lanes as 32 contiguous bytes.  Every
// load of a batch of 8 blocks is issued before any of them is used.
//
// The 16x16x32 bf16 matrix-core op multiplies the activations by the
// *unscaled* codebook values of one NF4 block (16 rows x 32 columns per op,
// two ops per block); the block's fp32 constant is then applied to the 4
// partial sums each lane holds (26. ..., Step 4: table[index] * scale, with
// the scale taken out of the 64-term sum it multiplies).  The codebook lookup
// goes through a byte -> bf16x2 table in LDS built from immediates.
//
// The rank-r pre-product u = x A^T is recomputed by every workgroup from the
// activation operand it already holds (extra 16x16x32 ops against rows of A,
// read from L2), so decode needs no second kernel and no grid-wide
// dependency.  Workgroup 0 stores u when the caller asks for it.
//
// Operand layout of v_mfma_f32_16x16x32_bf16 (gfx950): A lane l holds
// A[l % 16][8*(l/16) .. +8], B lane l holds B[8*(l/16) .. +8][l % 16], and the
// result lane l holds D[4*(l/16) .. +4][l % 16].  All operands use the same
// permutation of K within a block: op c of block b covers
// k = 64 b + 16 q + 8 c + e for lane group q = l / 16 and e = 0..7.
#include "kernels.h"

namespace qlora {

constexpr int kGemvRows = 16;
constexpr int kGemvWaves = 8;
// NF4 blocks whose loads are in flight together: 8 for a 16-wide rank tile
// in bf16, fewer as the per-block register footprint grows.
template <typename LT, int JT>
constexpr int gemv_batch() {
  constexpr int w = JT * (int)(sizeof(LT) / 2);
  return w >= 8 ? 1 : 8 / w;
}

__device__ __forceinline__ float nf4_immediate(int i) {
  constexpr float cb[16] = QL_NF4_CODEBOOK_VALUES;
  float v = cb[0];
#pragma unroll
  for (int k = 1; k < 16; ++k) v = (i == k) ? cb[k] : v;
  return v;
}

// 16 consecutive LoRA-A values of one rank row, kept raw until use.
template <typename LT>
struct ARaw;
template <>
struct ARaw<uint16_t> {
  u32x4 v[2];
  __device__ __forceinline__ void load(const uint16_t *p) {
    v[0] = reinterpret_cast<const u32x4 *>(p)[0];
    v[1] = reinterpret_cast<const u32x4 *>(p)[1];
  }
  __device__ __forceinline__ u32x4 half(int c) const { return v[c]; }
};
template <>
struct ARaw<float> {
  float4 v[4];
  __device__ __forceinline__ void load(const float *p) {
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = reinterpret_cast<const float4 *>(p)[i];
  }
  __device__ __forceinline__ u32x4 half(int c) const {
    const float4 a = v[2 * c], b = v[2 * c + 1];
    return u32x4{pack_bf16x2(a.x, a.y), pack_bf16x2(a.z, a.w), pack_bf16x2(b.x, b.y),
                 pack_bf16x2(b.z, b.w)};
  }
};

template <typename LT, int JT>
struct GemvBlock {
  u32x2 w;        // 16 packed indices of this lane's row
  int q8;         // double-quantisation code (or unused)
  float sg;       // its second-level scale, or the fp32 absmax
  u32x4 x0, x1;   // 2 x 8 activations
  ARaw<LT> a[JT]; // LoRA A rows 16 jt + l % 16
};

template <typename LT, int JT, bool DQ>
__global__ __launch_bounds__(512) void k_gemv_fwd(const uint16_t *__restrict__ x, int M,
                                                  const uint8_t *__restrict__ packed,
                                                  BlockScales sc, int64_t N, int64_t K,
                                                  const LT *__restrict__ A,
                                                  const LT *__restrict__ B, int32_t r, float s,
                                                  uint16_t *__restrict__ y,
                                                  float *__restrict__ u_save) {
  __shared__ uint32_t lut[256];
  __shared__ float red[kGemvWaves][16][16];
  __shared__ float ured[kGemvWaves][16][16 * JT];
  __shared__ float us[16][16 * JT];
  __shared__ float bs[16][16 * JT];
  const int t = threadIdx.x;
  const int wave = t >> 6, lane = t & 63;
  const int nl = lane & 15, q = lane >> 4;
  const int64_t n0 = (int64_t)blockIdx.x * kGemvRows;
  // Rows past N, token rows past M and rank rows past r are clamped to valid
  // ones: they only produce outputs that are never stored or summed.
  const int64_t n = n0 + nl < N ? n0 + nl : N - 1;
  const int m = nl < M ? nl : M - 1;
  const int64_t KB = K >> 6;
  const int64_t bpw = (KB + kGemvWaves - 1) / kGemvWaves;
  const int64_t b_begin = wave * bpw < KB ? wave * bpw : KB;
  const int64_t b_end = b_begin + bpw < KB ? b_begin + bpw : KB;
  const uint8_t *wrow = packed + ((n * K) >> 1) + 8 * q;
  const uint16_t *xrow = x + (int64_t)m * K + 16 * q;
  const LT *arow[JT];
#pragma unroll
  for (int jt = 0; jt < JT; ++jt) {
    const int j = 16 * jt + nl < r ? 16 * jt + nl : r - 1;
    arow[jt] = A + (int64_t)j * K + 16 * q;
  }
  const int64_t sbase = n * KB;
  const float mu = DQ ? sc.mu[0] : 0.0f;

  constexpr int kGemvBatch = gemv_batch<LT, JT>();
  GemvBlock<LT, JT> bl[kGemvBatch];
  auto load_batch = [&](int64_t b0, int cnt) {
#pragma unroll
    for (int i = 0; i < kGemvBatch; ++i) {
      if (i < cnt) {
        const int64_t b = b0 + i;
        bl[i].w = *reinterpret_cast<const u32x2 *>(wrow + 32 * b);
        if constexpr (DQ) {
          bl[i].q8 = sc.q[sbase + b];
          bl[i].sg = sc.sigma[(sbase + b) >> 8];
        } else {
          bl[i].q8 = 0;
          bl[i].sg = sc.absmax[sbase + b];
        }
        const u32x4 *xp = reinterpret_cast<const u32x4 *>(xrow + 64 * b);
        bl[i].x0 = xp[0];
        bl[i].x1 = xp[1];
#pragma unroll
        for (int jt = 0; jt < JT; ++jt) bl[i].a[jt].load(arow[jt] + 64 * b);
      }
    }
  };

  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  f32x4 uacc[JT];
#pragma unroll
  for (int jt = 0; jt < JT; ++jt) uacc[jt] = f32x4{0.f, 0.f, 0.f, 0.f};

  int64_t b0 = b_begin;
  int cnt = (int)(b_end - b0 < kGemvBatch ? b_end - b0 : kGemvBatch);
  load_batch(b0, cnt);
  // while the first loads are in flight: codebook table and this
  // workgroup's rows of B
  if (t < 256) {
    const uint16_t hi = f32_to_bf16_bits(nf4_immediate(t >> 4));
    const uint16_t lo = f32_to_bf16_bits(nf4_immediate(t & 15));
    lut[t] = (uint32_t)hi | ((uint32_t)lo << 16);
  }
  for (int e = t; e < 16 * 16 * JT; e += 512) {
    const int row = e / (16 * JT), j = e % (16 * JT);
    const int64_t nn = n0 + row < N ? n0 + row : N - 1;
    bs[row][j] = j < r ? load_as_f32(B, nn * r + j) : 0.0f;
  }
  __syncthreads();

  while (cnt > 0) {
#pragma unroll
    for (int i = 0; i < kGemvBatch; ++i) {
      if (i < cnt) {
        const GemvBlock<LT, JT> &g = bl[i];
        u32x4 wb0, wb1;
        wb0.x = lut[g.w.x & 0xFF];
        wb0.y = lut[(g.w.x >> 8) & 0xFF];
        wb0.z = lut[(g.w.x >> 16) & 0xFF];
        wb0.w = lut[g.w.x >> 24];
        wb1.x = lut[g.w.y & 0xFF];
        wb1.y = lut[(g.w.y >> 8) & 0xFF];
        wb1.z = lut[(g.w.y >> 16) & 0xFF];
        wb1.w = lut[g.w.y >> 24];
        const bf16x8 xa0 = __builtin_bit_cast(bf16x8, g.x0);
        const bf16x8 xa1 = __builtin_bit_cast(bf16x8, g.x1);
        f32x4 part = {0.f, 0.f, 0.f, 0.f};
        part = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa0, __builtin_bit_cast(bf16x8, wb0), part,
                                                       0, 0, 0);
        part = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa1, __builtin_bit_cast(bf16x8, wb1), part,
                                                       0, 0, 0);
        // part[v] = sum over the block of x[4q+v][k] * cb[idx[n][k]] for column n = n0 + nl
        const float a = DQ ? __builtin_fmaf((float)g.q8, g.sg, mu) : g.sg;
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[v] = __builtin_fmaf(a, part[v], acc[v]);
#pragma unroll
        for (int jt = 0; jt < JT; ++jt) {
          uacc[jt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              xa0, __builtin_bit_cast(bf16x8, g.a[jt].half(0)), uacc[jt], 0, 0, 0);
          uacc[jt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              xa1, __builtin_bit_cast(bf16x8, g.a[jt].half(1)), uacc[jt], 0, 0, 0);
        }
      }
    }
    b0 += kGemvBatch;
    cnt = (int)(b_end - b0 < kGemvBatch ? (b_end - b0 > 0 ? b_end - b0 : 0) : kGemvBatch);
    if (cnt > 0) load_batch(b0, cnt);
  }

  // D[4q + v][nl]: y partials per (m, n) and u partials per (m, j)
#pragma unroll
  for (int v = 0; v < 4; ++v) red[wave][4 * q + v][nl] = acc[v];
#pragma unroll
  for (int jt = 0; jt < JT; ++jt)
#pragma unroll
    for (int v = 0; v < 4; ++v) ured[wave][4 * q + v][16 * jt + nl] = uacc[jt][v];
  __syncthreads();
  for (int e = t; e < 16 * 16 * JT; e += 512) {
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
      y[(int64_t)mo * N + nn] = f32_to_bf16_bits(__builtin_fmaf(s, l, sum));
    }
  }
}

template <typename LT, int JT>
static void launch_jt(dim3 grid, hipStream_t stream, const uint16_t *x, int M,
                      const uint8_t *packed, BlockScales sc, int64_t N, int64_t K, const void *A,
                      const void *B, int32_t r, float s, uint16_t *y, float *u_save) {
  if (sc.absmax == nullptr)
    hipLaunchKernelGGL((k_gemv_fwd<LT, JT, true>), grid, dim3(512), 0, stream, x, M, packed, sc, N,
                       K, (const LT *)A, (const LT *)B, r, s, y, u_save);
  else
    hipLaunchKernelGGL((k_gemv_fwd<LT, JT, false>), grid, dim3(512), 0, stream, x, M, packed, sc,
                       N, K, (const LT *)A, (const LT *)B, r, s, y, u_save);
}

template <typename LT>
static void launch_lt(dim3 grid, hipStream_t stream, const uint16_t *x, int M,
                      const uint8_t *packed, BlockScales sc, int64_t N, int64_t K, const void *A,
                      const void *B, int32_t r, float s, uint16_t *y, float *u_save) {
  if (r <= 16) launch_jt<LT, 1>(grid, stream, x, M, packed, sc, N, K, A, B, r, s, y, u_save);
  else if (r <= 32) launch_jt<LT, 2>(grid, stream, x, M, packed, sc, N, K, A, B, r, s, y, u_save);
  else if (r <= 64) launch_jt<LT, 4>(grid, stream, x, M, packed, sc, N, K, A, B, r, s, y, u_save);
  else launch_jt<LT, 8>(grid, stream, x, M, packed, sc, N, K, A, B, r, s, y, u_save);
}

int launch_gemv_fwd(const uint16_t *x, int64_t M, const uint8_t *packed, BlockScales sc,
                    int64_t N, int64_t K, const void *A, const void *B, int lora_dtype, int32_t r,
                    float s, uint16_t *y, float *u_save, hipStream_t stream) {
  const dim3 grid((unsigned)((N + kGemvRows - 1) / kGemvRows));
  if (lora_dtype == QL_BF16)
    launch_lt<uint16_t>(grid, stream, x, (int)M, packed, sc, N, K, A, B, r, s, y, u_save);
  else
    launch_lt<float>(grid, stream, x, (int)M, packed, sc, N, K, A, B, r, s, y, u_save);
  QL_HIP_CHECK_LAUNCH();
  return QL_OK;
}

}  // namespace qlora
