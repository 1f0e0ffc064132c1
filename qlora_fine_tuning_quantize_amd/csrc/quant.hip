// quant.hip -- NF4 quantisation, double quantisation and dequantisation
// kernels for gfx950.
//
// Method (Gemma lesson 09 "QLoRA 4-bit quantised fine-tuning", sec. 9.2.1):
// split the flattened weight into blocks, normalise each block to [-1, 1] by
// its absolute maximum, map every value to the nearest NF4 codepoint and
// store the 4-bit index (two per byte: 22. QLoRA and 4bit Quantization,
// Step 4).  Sec. 9.2.2: the block constants are quantised again to 8-bit
// integers (double quantisation).  Dequantisation is table[index] * scale
// (26. QLoRA and 4bit Quantization, Step 4).
#include <math.h>

#include "kernels.h"

namespace qlora {

static const float kCodebookHost[16] = QL_NF4_CODEBOOK_VALUES;

const float *nf4_codebook_host() { return kCodebookHost; }

NF4Thresholds nf4_thresholds() {
  float t[15];
  for (int i = 0; i < 15; ++i) {
    // The midpoint of two fp32 values is exact in fp64; round it down to fp32.
    double mid = ((double)kCodebookHost[i] + (double)kCodebookHost[i + 1]) * 0.5;
    float v = (float)mid;
    if ((double)v > mid) v = nextafterf(v, -INFINITY);
    t[i] = v;
  }
  return NF4Thresholds{t[0], t[1], t[2],  t[3],  t[4],  t[5],  t[6], t[7],
                       t[8], t[9], t[10], t[11], t[12], t[13], t[14]};
}

// Nearest-codepoint search.  The index of v is the number of thresholds
// below it.  [-1, 1] is cut into 64 buckets of width 1/32 (plus one for
// v == 1); the thresholds are at least 0.08 apart, so a bucket holds at most
// one of them, and no threshold lies within 2e-3 of a bucket edge.  Entry k
// stores c_k = number of thresholds below the bucket and t_k = the threshold
// inside it (+inf if none): index = c_k + (v > t_k).  The key
// trunc(fma(v, 32, 32)) is off by one only within ~1e-7 of an edge, where
// both neighbouring entries give the same index.
struct BucketEntry {
  int c;
  float t;
};
constexpr int kBuckets = 65;

__device__ __forceinline__ void build_buckets(BucketEntry *tab, const NF4Thresholds &th, int t) {
  if (t < kBuckets) {
    const float lo = -1.0f + (float)t * 0.03125f;
    const float hi = lo + 0.03125f;
    const float ts[15] = {th.t0, th.t1, th.t2,  th.t3,  th.t4,  th.t5,  th.t6, th.t7,
                          th.t8, th.t9, th.t10, th.t11, th.t12, th.t13, th.t14};
    int c = 0;
    float inside = __builtin_huge_valf();
#pragma unroll
    for (int i = 0; i < 15; ++i) {
      c += ts[i] < lo;
      if (ts[i] >= lo && ts[i] < hi) inside = ts[i];
    }
    tab[t] = BucketEntry{c, inside};
  }
}

__device__ __forceinline__ uint32_t nf4_index(float v, const BucketEntry *tab) {
  int key = (int)__builtin_fmaf(v, 32.0f, 32.0f);
  key = key < 0 ? 0 : (key > kBuckets - 1 ? kBuckets - 1 : key);
  const BucketEntry e = tab[key];
  return (uint32_t)e.c + (v > e.t ? 1u : 0u);
}

// ---------------------------------------------------------------------------
// K1: one NF4 block of 64 elements per group of 8 lanes; each lane loads 8
// consecutive elements (16 B of bf16), the group reduces |w| with
// cross-lane max, then each lane divides, searches and packs 8 nibbles into
// one 32-bit word.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void k_nf4_quantize(const T *__restrict__ w, int64_t n,
                                                      uint8_t *__restrict__ packed,
                                                      float *__restrict__ absmax,
                                                      NF4Thresholds th) {
  __shared__ BucketEntry tab[kBuckets];
  build_buckets(tab, th, threadIdx.x);
  __syncthreads();
  const int64_t gtid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t blk = gtid >> 3;
  const int64_t e0 = gtid * 8;
  float v[8];
  const bool full = e0 + 8 <= n;
  if (full) {
    if constexpr (sizeof(T) == 2) {
      uint4 raw = *reinterpret_cast<const uint4 *>(w + e0);
      uint32_t r[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[2 * i] = __uint_as_float(r[i] << 16);
        v[2 * i + 1] = __uint_as_float(r[i] & 0xFFFF0000u);
      }
    } else {
      float4 a = *reinterpret_cast<const float4 *>(w + e0);
      float4 b = *reinterpret_cast<const float4 *>(w + e0 + 4);
      v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
      v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = (e0 + i < n) ? load_as_f32(w, e0 + i) : 0.0f;
  }
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[i]));
  m = fmaxf(m, __shfl_xor(m, 1, 8));
  m = fmaxf(m, __shfl_xor(m, 2, 8));
  m = fmaxf(m, __shfl_xor(m, 4, 8));
  if (e0 >= n) return;  // after the group reduction: lanes past the end only helped
  uint32_t word = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    uint32_t idx = 7;
    if (m != 0.0f) idx = nf4_index(v[i] / m, tab);
    if (e0 + i < n) word |= idx << ((i & 1) ? 8 * (i >> 1) : 8 * (i >> 1) + 4);
  }
  if (full) {
    *reinterpret_cast<uint32_t *>(packed + (e0 >> 1)) = word;
  } else {
    for (int j = 0; j < 4; ++j)
      if (e0 + 2 * j < n) packed[(e0 >> 1) + j] = (uint8_t)(word >> (8 * j));
  }
  if ((threadIdx.x & 7) == 0) absmax[blk] = m;
}

// ---------------------------------------------------------------------------
// K2: fixed-order fp64 partial sums of the block constants, 8192 per
// workgroup (each lane sums 32 consecutive values in index order, then a
// fixed binary tree over the 256 lanes).
// ---------------------------------------------------------------------------
constexpr int kDqSumChunk = 8192;

__global__ __launch_bounds__(256) void k_dq_partial_sums(const float *__restrict__ a, int64_t nb,
                                                         double *__restrict__ partial) {
  __shared__ double sh[256];
  const int64_t base = (int64_t)blockIdx.x * kDqSumChunk + threadIdx.x * 32;
  double s = 0.0;
  for (int i = 0; i < 32; ++i)
    if (base + i < nb) s += (double)a[base + i];
  sh[threadIdx.x] = s;
  __syncthreads();
  for (int stride = 128; stride > 0; stride >>= 1) {
    if (threadIdx.x < stride) sh[threadIdx.x] += sh[threadIdx.x + stride];
    __syncthreads();
  }
  if (threadIdx.x == 0) partial[blockIdx.x] = sh[0];
}

// ---------------------------------------------------------------------------
// K3: one workgroup per 256 block constants.  Every workgroup first reduces
// the partial sums in the same fixed order, so all agree on mu.  Then
// d = a - mu, sigma = max|d| / 127, code = clamp(rint(d / sigma), +-127).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_dq_codes(const float *__restrict__ a, int64_t nb,
                                                  const double *__restrict__ partial, int n_partial,
                                                  int8_t *__restrict__ q, float *__restrict__ sigma,
                                                  float *__restrict__ mean_out) {
  __shared__ double shd[256];
  __shared__ float shf[256];
  const int t = threadIdx.x;
  double s = 0.0;
  for (int i = t; i < n_partial; i += 256) s += partial[i];
  shd[t] = s;
  __syncthreads();
  for (int stride = 128; stride > 0; stride >>= 1) {
    if (t < stride) shd[t] += shd[t + stride];
    __syncthreads();
  }
  const float mu = (float)(shd[0] / (double)nb);
  const int64_t j = (int64_t)blockIdx.x * 256 + t;
  const float d = (j < nb) ? a[j] - mu : 0.0f;
  shf[t] = fabsf(d);
  __syncthreads();
  for (int stride = 128; stride > 0; stride >>= 1) {
    if (t < stride) shf[t] = fmaxf(shf[t], shf[t + stride]);
    __syncthreads();
  }
  const float sg = shf[0] / 127.0f;
  if (j < nb) {
    float c = 0.0f;
    if (sg != 0.0f) {
      c = __builtin_rintf(d / sg);
      c = fminf(fmaxf(c, -127.0f), 127.0f);
    }
    q[j] = (int8_t)(int)c;
  }
  if (t == 0) {
    sigma[blockIdx.x] = sg;
    if (blockIdx.x == 0) mean_out[0] = mu;
  }
}

// ---------------------------------------------------------------------------
// K4: dequantisation.  Each lane expands 16 packed bytes (32 elements, half
// an NF4 block) through a byte -> (cb[hi], cb[lo]) table in LDS and scales by
// the block constant.
// ---------------------------------------------------------------------------
template <typename OutT>
__global__ __launch_bounds__(256) void k_nf4_dequantize(const uint8_t *__restrict__ packed,
                                                        int64_t n, BlockScales sc,
                                                        OutT *__restrict__ out) {
  __shared__ float2 lut[256];
  lut[threadIdx.x] = make_float2(c_nf4[threadIdx.x >> 4], c_nf4[threadIdx.x & 15]);
  __syncthreads();
  const int64_t gtid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t e0 = gtid * 32;
  if (e0 >= n) return;
  const float a = sc(e0 >> 6);
  if (e0 + 32 <= n) {
    uint4 raw = *reinterpret_cast<const uint4 *>(packed + (e0 >> 1));
    uint32_t r[4] = {raw.x, raw.y, raw.z, raw.w};
    float o[32];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float2 p = lut[(r[i >> 2] >> (8 * (i & 3))) & 0xFF];
      o[2 * i] = p.x * a;
      o[2 * i + 1] = p.y * a;
    }
    if constexpr (sizeof(OutT) == 2) {
      uint32_t pk[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) pk[i] = pack_bf16x2(o[2 * i], o[2 * i + 1]);
      uint4 *dst = reinterpret_cast<uint4 *>(out + e0);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        dst[i] = make_uint4(pk[4 * i], pk[4 * i + 1], pk[4 * i + 2], pk[4 * i + 3]);
    } else {
      float4 *dst = reinterpret_cast<float4 *>(out + e0);
#pragma unroll
      for (int i = 0; i < 8; ++i)
        dst[i] = make_float4(o[4 * i], o[4 * i + 1], o[4 * i + 2], o[4 * i + 3]);
    }
  } else {
    for (int64_t i = e0; i < n; ++i) {
      uint8_t byte = packed[i >> 1];
      uint32_t idx = (i & 1) ? (byte & 15u) : (byte >> 4);
      store_from_f32(out, i, c_nf4[idx] * a);
    }
  }
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
int launch_nf4_quantize(const void *w, int w_dtype, int64_t n, uint8_t *packed, float *absmax,
                        hipStream_t stream) {
  if (n <= 0) return QL_OK;
  const int64_t threads = (n + 7) / 8;
  const dim3 grid((unsigned)((threads + 255) / 256));
  const NF4Thresholds th = nf4_thresholds();
  if (w_dtype == QL_BF16)
    hipLaunchKernelGGL(k_nf4_quantize<uint16_t>, grid, dim3(256), 0, stream,
                       (const uint16_t *)w, n, packed, absmax, th);
  else
    hipLaunchKernelGGL(k_nf4_quantize<float>, grid, dim3(256), 0, stream, (const float *)w, n,
                       packed, absmax, th);
  QL_HIP_CHECK_LAUNCH();
  return QL_OK;
}

size_t dq_partial_count(int64_t nb) { return (size_t)((nb + kDqSumChunk - 1) / kDqSumChunk); }

int launch_double_quant(const float *absmax, int64_t nb, double *partial, int8_t *q, float *sigma,
                        float *mean_out, hipStream_t stream) {
  if (nb <= 0) return QL_OK;
  const int np = (int)dq_partial_count(nb);
  hipLaunchKernelGGL(k_dq_partial_sums, dim3(np), dim3(256), 0, stream, absmax, nb, partial);
  QL_HIP_CHECK_LAUNCH();
  const unsigned nb2 = (unsigned)((nb + 255) / 256);
  hipLaunchKernelGGL(k_dq_codes, dim3(nb2), dim3(256), 0, stream, absmax, nb, partial, np, q,
                     sigma, mean_out);
  QL_HIP_CHECK_LAUNCH();
  return QL_OK;
}

int launch_nf4_dequantize(const uint8_t *packed, int64_t n, BlockScales sc, void *out,
                          int out_dtype, hipStream_t stream) {
  if (n <= 0) return QL_OK;
  const int64_t threads = (n + 31) / 32;
  const dim3 grid((unsigned)((threads + 255) / 256));
  if (out_dtype == QL_BF16)
    hipLaunchKernelGGL(k_nf4_dequantize<uint16_t>, grid, dim3(256), 0, stream, packed, n, sc,
                       (uint16_t *)out);
  else
    hipLaunchKernelGGL(k_nf4_dequantize<float>, grid, dim3(256), 0, stream, packed, n, sc,
                       (float *)out);
  QL_HIP_CHECK_LAUNCH();
  return QL_OK;
}

}  // namespace qlora
