// gemv.hip -- decode-sized forward of the QLoRA layer (M <= 16 tokens, bf16).
//
//   y = x W^^T + s u B^T        (26. QLoRA and 4bit Quantization, Step 3)
//
// Memory-bound: the packed 4-bit weight is the dominant traffic.  Each
// workgroup owns 16 weight rows; its 8 waves split the K dimension.  A lane
// of a wave holds 16 consecutive indices (8 bytes) of one row per NF4 block,
// so one block of one row is read by 4 lanes as 32 contiguous bytes.
//
// The 16x16x32 bf16 matrix-core op multiplies the activations by the
// *unscaled* codebook values of one NF4 block (16 rows x 32 columns per op,
// two ops per block); the block's fp32 constant is then applied to the 4
// partial sums each lane holds (26. ..., Step 4: table[index] * scale, with
// the scale taken out of the 64-term sum it multiplies).  The codebook lookup
// goes through a byte -> bf16x2 table in LDS.
//
// Operand layout of v_mfma_f32_16x16x32_bf16 (gfx950): A lane l holds
// A[l % 16][8*(l/16) .. +8], B lane l holds B[8*(l/16) .. +8][l % 16], and the
// result lane l holds D[4*(l/16) .. +4][l % 16].  Both operands use the same
// permutation of K within a block: MFMA c of block b covers
// k = 64 b + 16 q + 8 c + e for lane group q = l / 16 and e = 0..7.
#include "kernels.h"

namespace qlora {

constexpr int kGemvRows = 16;
constexpr int kGemvWaves = 8;
constexpr int kGemvBatch = 8;  // NF4 blocks whose loads are all in flight together

// u is passed as S partial sums [S][M][r] of the rank-r pre-product; the
// epilogue adds them in slice order (the same order as the stand-alone
// reduction) before applying the bypass.
template <typename LT>
__global__ __launch_bounds__(512) void k_gemv_fwd(const uint16_t *__restrict__ x, int M,
                                                  const uint8_t *__restrict__ packed,
                                                  BlockScales sc, int64_t N, int64_t K,
                                                  const float *__restrict__ u_part, int S,
                                                  const LT *__restrict__ B, int32_t r, float s,
                                                  uint16_t *__restrict__ y) {
  __shared__ uint32_t lut[256];
  __shared__ float red[kGemvWaves][16][16];
  __shared__ float us[16][128];
  const int t = threadIdx.x;
  if (t < 256) {
    const uint16_t hi = f32_to_bf16_bits(c_nf4[t >> 4]);
    const uint16_t lo = f32_to_bf16_bits(c_nf4[t & 15]);
    lut[t] = (uint32_t)hi | ((uint32_t)lo << 16);
  }

  const int wave = t >> 6, lane = t & 63;
  const int nl = lane & 15, q = lane >> 4;
  const int64_t n0 = (int64_t)blockIdx.x * kGemvRows;
  const int64_t n = n0 + nl;
  const bool row_ok = n < N;
  const int m = nl;  // the A-operand row this lane supplies
  const int64_t KB = K >> 6;
  const int64_t bpw = (KB + kGemvWaves - 1) / kGemvWaves;
  const int64_t b_begin = wave * bpw;
  const int64_t b_end = b_begin + bpw < KB ? b_begin + bpw : KB;
  const uint8_t *wrow = packed + ((n * K) >> 1) + 8 * q;
  const uint16_t *xrow = x + (int64_t)m * K + 16 * q;
  const int64_t sbase = n * KB;
  const float mu = sc.absmax ? 0.0f : sc.mu[0];
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  __syncthreads();  // lut

  for (int64_t b0 = b_begin; b0 < b_end; b0 += kGemvBatch) {
    u32x2 wq[kGemvBatch];
    float a[kGemvBatch];
    u32x4 xa[kGemvBatch][2];
#pragma unroll
    for (int i = 0; i < kGemvBatch; ++i) {
      const int64_t b = b0 + i;
      const bool ok = b < b_end;
      wq[i] = u32x2{0u, 0u};
      a[i] = 0.0f;
      if (row_ok && ok) {
        wq[i] = *reinterpret_cast<const u32x2 *>(wrow + 32 * b);
        a[i] = sc.absmax ? sc.absmax[sbase + b]
                         : __builtin_fmaf((float)sc.q[sbase + b], sc.sigma[(sbase + b) >> 8], mu);
      }
      xa[i][0] = u32x4{0u, 0u, 0u, 0u};
      xa[i][1] = u32x4{0u, 0u, 0u, 0u};
      if (m < M && ok) {
        const u32x4 *xp = reinterpret_cast<const u32x4 *>(xrow + 64 * b);
        xa[i][0] = xp[0];
        xa[i][1] = xp[1];
      }
    }
#pragma unroll
    for (int i = 0; i < kGemvBatch; ++i) {
      u32x4 wb0, wb1;
      wb0.x = lut[wq[i].x & 0xFF];
      wb0.y = lut[(wq[i].x >> 8) & 0xFF];
      wb0.z = lut[(wq[i].x >> 16) & 0xFF];
      wb0.w = lut[wq[i].x >> 24];
      wb1.x = lut[wq[i].y & 0xFF];
      wb1.y = lut[(wq[i].y >> 8) & 0xFF];
      wb1.z = lut[(wq[i].y >> 16) & 0xFF];
      wb1.w = lut[wq[i].y >> 24];
      f32x4 part = {0.f, 0.f, 0.f, 0.f};
      part = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, xa[i][0]),
                                                     __builtin_bit_cast(bf16x8, wb0), part, 0, 0, 0);
      part = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, xa[i][1]),
                                                     __builtin_bit_cast(bf16x8, wb1), part, 0, 0, 0);
      // part[v] = sum over the block of x[4q+v][k] * cb[idx[n][k]] for column n = n0 + nl
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[v] = __builtin_fmaf(a[i], part[v], acc[v]);
    }
  }
  // D[4q + v][nl] -> red[wave][m][n]
#pragma unroll
  for (int v = 0; v < 4; ++v) red[wave][4 * q + v][nl] = acc[v];
  for (int e = t; e < M * r; e += 512) {
    const int mo = e / r, j = e % r;
    float uj = 0.0f;
    for (int si = 0; si < S; ++si) uj += u_part[((int64_t)si * M + mo) * r + j];
    us[mo][j] = uj;
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
      for (int j = 0; j < r; ++j) l = __builtin_fmaf(us[mo][j], load_as_f32(B, nn * r + j), l);
      y[(int64_t)mo * N + nn] = f32_to_bf16_bits(__builtin_fmaf(s, l, sum));
    }
  }
}

int launch_gemv_fwd(const uint16_t *x, int64_t M, const uint8_t *packed, BlockScales sc,
                    int64_t N, int64_t K, const float *u_part, int S, const void *B,
                    int lora_dtype, int32_t r, float s, uint16_t *y, hipStream_t stream) {
  const dim3 grid((unsigned)((N + kGemvRows - 1) / kGemvRows));
  if (lora_dtype == QL_BF16)
    hipLaunchKernelGGL(k_gemv_fwd<uint16_t>, grid, dim3(512), 0, stream, x, (int)M, packed, sc, N,
                       K, u_part, S, (const uint16_t *)B, r, s, y);
  else
    hipLaunchKernelGGL(k_gemv_fwd<float>, grid, dim3(512), 0, stream, x, (int)M, packed, sc, N, K,
                       u_part, S, (const float *)B, r, s, y);
  QL_HIP_CHECK_LAUNCH();
  return QL_OK;
}

}  // namespace qlora
