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
// one of them, and no threshold lies within 1.9e-3 of a bucket edge.  Entry k
// stores c_k = number of thresholds below the bucket and t_k = the threshold
// inside it (+inf if none): index = c_k + (v > t_k).  The key
// trunc(fma(v, 32, 32)) is off by one only within ~1e-7 of an edge, where
// both neighbouring entries give the same index.  g_k is the half-width of
// a guard band |v - t_k| < g_k of relative width 2^-20 around t_k (0 when
// there is no threshold), used by the reciprocal fast path below.
struct BucketEntry {
  int c;
  float t, g, pad;
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
    const float g = inside != __builtin_huge_valf() ? fabsf(inside) * 0x1p-20f : 0.0f;
    tab[t] = BucketEntry{c, inside, g, 0.0f};
  }
}

__device__ __forceinline__ const BucketEntry &bucket_of(float v, const BucketEntry *tab) {
  int key = (int)__builtin_fmaf(v, 32.0f, 32.0f);
  key = key < 0 ? 0 : (key > kBuckets - 1 ? kBuckets - 1 : key);
  return tab[key];
}

__device__ __forceinline__ uint32_t nf4_index(float v, const BucketEntry *tab) {
  const BucketEntry &e = bucket_of(v, tab);
  return (uint32_t)e.c + (v > e.t ? 1u : 0u);
}

// The index of v' = w * r instead of v = RN(w / a), where r is the
// hardware reciprocal of a (v_rcp_f32, within 1 ulp of 1/a).  For a normal
// block maximum a in [2^-125, 2^125] (so 1/a is normal too), |v' - v| is at
// most ~3.5 ulp of v; the two give different indices only if a threshold
// lies between them or on one of them, i.e. only if v' falls inside the
// guard band (2^-20 relative, >= 8 ulp) around the threshold of its bucket.
// That case is flagged (as a wave mask of lanes, in `near`) and decided
// with the exact division.  |w| <= a gives |v'| <= 1 + 2^-23, so the bucket
// key needs no clamp.
__device__ __forceinline__ uint32_t nf4_index_fast(float vp, const BucketEntry *tab,
                                                   uint64_t &near) {
#pragma clang fp contract(off)  // the guard test is on the rounded v'
  const BucketEntry &e = tab[(int)__builtin_fmaf(vp, 32.0f, 32.0f)];
  near |= __builtin_amdgcn_ballot_w64(fabsf(vp - e.t) < e.g);
  return (uint32_t)e.c + (vp > e.t ? 1u : 0u);
}

// Max over the L = 8 or 16 lanes of an aligned group (DPP: swap neighbours,
// swap pairs, mirror within the group of 8, then for 16 mirror within the
// row of 16; every lane ends with the max).
template <int L>
__device__ __forceinline__ float max_lanes(float m) {
  const int qp_1032 = 0xB1, qp_2301 = 0x4E, row_half_mirror = 0x141, row_mirror = 0x140;
  m = fmaxf(m, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(m), qp_1032, 0xF,
                                                            0xF, true)));
  m = fmaxf(m, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(m), qp_2301, 0xF,
                                                            0xF, true)));
  m = fmaxf(m, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(m), row_half_mirror,
                                                            0xF, 0xF, true)));
  if constexpr (L == 16)
    m = fmaxf(m, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(m), row_mirror,
                                                              0xF, 0xF, true)));
  return m;
}

// ---------------------------------------------------------------------------
// K1: a wave owns 2 runs of 512 consecutive elements (8 NF4 blocks of 64,
// or 4 of 128); in every run lane l takes the 8 elements 8l .. 8l + 7, so
// each block is held by a group of BLK / 8 lanes and every load and store
// instruction of the wave covers one contiguous span.  All loads are issued first.  The group
// reduces |w| (DPP), then each lane finds its 8 indices and packs them into
// one 32-bit word.  The indices are those of the correctly rounded w / a:
// each lane takes a reciprocal of a once and the index of w times it; a lane with
// any element in a guard band (or with a block maximum outside the normal
// range) redoes its 8 elements with the division.
// ---------------------------------------------------------------------------
template <typename T, int BLK>
__global__ __launch_bounds__(256) void k_nf4_quantize(const T *__restrict__ w, int64_t n,
                                                      uint8_t *__restrict__ packed,
                                                      float *__restrict__ absmax,
                                                      NF4Thresholds th) {
  __shared__ BucketEntry tab[kBuckets];
  const int lane = threadIdx.x & 63;
  const int64_t wave = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 6;
  constexpr int R = 2;
  int64_t e0[R];
  float v[R][8];
#pragma unroll
  for (int j = 0; j < R; ++j) {
    e0[j] = wave * (R * 512) + j * 512 + lane * 8;
    // a run that is not whole loads from the start instead (n >= 8 there)
    // and is reloaded element by element below
    const int64_t ec = e0[j] + 8 <= n ? e0[j] : 0;
    if (n < 8) {  // uniform: too short for any 8-element load
#pragma unroll
      for (int i = 0; i < 8; ++i) v[j][i] = 0.0f;
    } else if constexpr (sizeof(T) == 2) {  // bf16 or fp16: widening is exact
      const u32x4 raw = *reinterpret_cast<const u32x4 *>(w + ec);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[j][2 * i] = Half<T>::lo(raw[i]);
        v[j][2 * i + 1] = Half<T>::hi(raw[i]);
      }
    } else {
      const f32x4 a = *reinterpret_cast<const f32x4 *>(w + ec);
      const f32x4 b = *reinterpret_cast<const f32x4 *>(w + ec + 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[j][i] = a[i];
        v[j][4 + i] = b[i];
      }
    }
  }
  build_buckets(tab, th, threadIdx.x);
  __syncthreads();
#pragma unroll
  for (int j = 0; j < R; ++j) {
    if (e0[j] + 8 > n) {  // the ragged end (or past it): elements past n count as 0
#pragma unroll
      for (int i = 0; i < 8; ++i) v[j][i] = (e0[j] + i < n) ? load_as_f32(w, e0[j] + i) : 0.0f;
    }
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[j][i]));
    m = max_lanes<BLK / 8>(m);
    if (e0[j] >= n) continue;  // after the group reduction: lanes past the end only helped
    // element i goes to byte i / 2, high nibble for even i
    uint32_t word = 0x77777777u;  // a zero block: every element is the exact zero
    if (m != 0.0f) {
      bool slow = !(m >= 0x1p-125f && m <= 0x1p125f);
      if (!slow) {
        const float rm = __builtin_amdgcn_rcpf(m);
        uint64_t near = 0;
        word = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i)
          word |= nf4_index_fast(v[j][i] * rm, tab, near)
                  << ((i & 1) ? 8 * (i >> 1) : 8 * (i >> 1) + 4);
        slow = (near >> lane) & 1u;
      }
      if (slow) {
        word = 0;
        for (int i = 0; i < 8; ++i)
          word |= nf4_index(v[j][i] / m, tab) << ((i & 1) ? 8 * (i >> 1) : 8 * (i >> 1) + 4);
      }
    }
    if (e0[j] + 8 <= n) {
      *reinterpret_cast<uint32_t *>(packed + (e0[j] >> 1)) = word;
    } else {
      // nibbles of elements past n are 0
      for (int i = 0; i < 8; ++i)
        if (e0[j] + i >= n) word &= ~(0xFu << ((i & 1) ? 8 * (i >> 1) : 8 * (i >> 1) + 4));
      for (int b = 0; b < 4; ++b)
        if (e0[j] + 2 * b < n) packed[(e0[j] >> 1) + b] = (uint8_t)(word >> (8 * b));
    }
    if ((lane & (BLK / 8 - 1)) == 0) absmax[e0[j] / BLK] = m;
  }
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
  float v[32];
  if (base + 32 <= nb) {  // 8 loads of 16 bytes, all in flight before the sum
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const f32x4 q = *reinterpret_cast<const f32x4 *>(a + base + 4 * i);
      v[4 * i] = q[0]; v[4 * i + 1] = q[1]; v[4 * i + 2] = q[2]; v[4 * i + 3] = q[3];
    }
  } else {
#pragma unroll
    for (int i = 0; i < 32; ++i) v[i] = base + i < nb ? a[base + i] : 0.0f;
  }
  double s = 0.0;
#pragma unroll
  for (int i = 0; i < 32; ++i) s += (double)v[i];
  sh[threadIdx.x] = s;
  __syncthreads();
  for (int stride = 128; stride > 0; stride >>= 1) {
    if (threadIdx.x < stride) sh[threadIdx.x] += sh[threadIdx.x + stride];
    __syncthreads();
  }
  if (threadIdx.x == 0) partial[blockIdx.x] = sh[0];
}

// ---------------------------------------------------------------------------
// K3: one wave per 256 block constants (4 per lane), 4 waves per workgroup.
// Every wave first reduces the partial sums in the same fixed order (lane l
// sums partials l, l + 64, ... in increasing order, then a fixed tree over
// the 64 lanes whose result lane 0 broadcasts), so all agree on mu.  Then
// d = a - mu, sigma = max|d| / 127, code = clamp(rint(d / sigma), +-127).
// ---------------------------------------------------------------------------
__device__ __forceinline__ double shfl_down_f64(double v, int delta) {
  const int lo = __shfl_down(__double2loint(v), delta, 64);
  const int hi = __shfl_down(__double2hiint(v), delta, 64);
  return __hiloint2double(hi, lo);
}

__global__ __launch_bounds__(256) void k_dq_codes(const float *__restrict__ a, int64_t nb,
                                                  const double *__restrict__ partial, int n_partial,
                                                  int8_t *__restrict__ q, float *__restrict__ sigma,
                                                  float *__restrict__ mean_out) {
  const int lane = threadIdx.x & 63;
  const int64_t b2 = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);  // this wave's DQ block
  const int64_t j0 = b2 * 256 + 4 * lane;
  // the lane's 4 constants (issued before the partial sums are reduced)
  float av[4];
  const bool full = j0 + 4 <= nb;
  if (full) {
    const f32x4 t = *reinterpret_cast<const f32x4 *>(a + j0);
    av[0] = t[0]; av[1] = t[1]; av[2] = t[2]; av[3] = t[3];
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) av[i] = j0 + i < nb ? a[j0 + i] : 0.0f;
  }
  double s = 0.0;
  for (int i = lane; i < n_partial; i += 64) s += partial[i];
#pragma unroll
  for (int delta = 32; delta > 0; delta >>= 1) s += shfl_down_f64(s, delta);
  s = __hiloint2double(__shfl(__double2hiint(s), 0, 64), __shfl(__double2loint(s), 0, 64));
  const float mu = (float)(s / (double)nb);
  if (b2 * 256 >= nb) return;  // after the wave-wide steps: a wave past the end only helped
  float d[4], amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    d[i] = j0 + i < nb ? av[i] - mu : 0.0f;
    amax = fmaxf(amax, fabsf(d[i]));
  }
#pragma unroll
  for (int delta = 32; delta > 0; delta >>= 1) amax = fmaxf(amax, __shfl_xor(amax, delta, 64));
  const float sg = amax / 127.0f;
  uint32_t word = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float c = 0.0f;
    if (sg != 0.0f) {
      c = __builtin_rintf(d[i] / sg);
      c = fminf(fmaxf(c, -127.0f), 127.0f);
    }
    word |= ((uint32_t)(int)c & 0xFFu) << (8 * i);
  }
  if (full && ((uintptr_t)q & 3u) == 0) {
    *reinterpret_cast<uint32_t *>(q + j0) = word;
  } else {  // ragged end, or a code array without 4-byte alignment
    for (int i = 0; i < 4; ++i)
      if (j0 + i < nb) q[j0 + i] = (int8_t)(word >> (8 * i));
  }
  if (lane == 0) {
    sigma[b2] = sg;
    if (b2 == 0) mean_out[0] = mu;
  }
}

// ---------------------------------------------------------------------------
// K4: dequantisation.  Every store is 16 bytes per lane (E = 8 bf16 / fp16 or 4
// fp32 elements) and every wave instruction covers one contiguous span: a
// wave owns 4 x 64 x E consecutive elements and lane l takes elements
// l E .. l E + E - 1 of each of its 4 runs of 64 E.  The E / 2 packed bytes
// of a run go through a byte -> (cb[hi], cb[lo]) table in LDS and are
// scaled by their block constant.  All loads of a lane are issued before
// any is used (out-of-range runs load from the start of the arrays and are
// not stored).
// ---------------------------------------------------------------------------
template <typename OutT>
__global__ __launch_bounds__(256) void k_nf4_dequantize(const uint8_t *__restrict__ packed,
                                                        int64_t n, BlockScales sc,
                                                        OutT *__restrict__ out) {
  constexpr int E = 16 / (int)sizeof(OutT);
  __shared__ float2 lut[256];
  lut[threadIdx.x] = make_float2(c_nf4[threadIdx.x >> 4], c_nf4[threadIdx.x & 15]);
  const int lane = threadIdx.x & 63;
  const int64_t wave = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 6;
  int64_t e[4];
  uint32_t raw[4];
  float a[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    e[i] = wave * (4 * 64 * E) + (int64_t)i * (64 * E) + lane * E;
    // a run that is not whole loads from the start instead (n >= E there)
    // and is stored element by element below
    const int64_t ec = e[i] + E <= n ? e[i] : 0;
    if (n < E)  // uniform: too short for any vector load
      raw[i] = 0;
    else if constexpr (E == 8)
      raw[i] = *reinterpret_cast<const uint32_t *>(packed + (ec >> 1));
    else
      raw[i] = *reinterpret_cast<const uint16_t *>(packed + (ec >> 1));
    a[i] = sc(ec >> 6);
  }
  __syncthreads();  // lut
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (e[i] + E <= n) {
      float o[E];
#pragma unroll
      for (int b = 0; b < E / 2; ++b) {
        const float2 p = lut[(raw[i] >> (8 * b)) & 0xFF];
        o[2 * b] = p.x * a[i];
        o[2 * b + 1] = p.y * a[i];
      }
      if constexpr (E == 8) {
        *reinterpret_cast<u32x4 *>(out + e[i]) =
            u32x4{Half<OutT>::pack2(o[0], o[1]), Half<OutT>::pack2(o[2], o[3]),
                  Half<OutT>::pack2(o[4], o[5]), Half<OutT>::pack2(o[6], o[7])};
      } else {
        *reinterpret_cast<f32x4 *>(out + e[i]) = f32x4{o[0], o[1], o[2], o[3]};
      }
    } else if (e[i] < n) {
      const float ai = sc(e[i] >> 6);
      for (int64_t k = e[i]; k < n; ++k) {
        const uint8_t byte = packed[k >> 1];
        const uint32_t idx = (k & 1) ? (byte & 15u) : (byte >> 4);
        store_from_f32(out, k, c_nf4[idx] * ai);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
int launch_nf4_quantize(const void *w, int w_dtype, int64_t n, int block, uint8_t *packed,
                        float *absmax, hipStream_t stream) {
  if (n <= 0) return QL_OK;
  // one wave per 1024 elements (2 runs of 512)
  const int64_t waves = (n + 1023) / 1024;
  const dim3 grid((unsigned)((waves + 3) / 4));
  const NF4Thresholds th = nf4_thresholds();
#define QL_QUANT(T, BLKV)                                                                        \
  hipLaunchKernelGGL((k_nf4_quantize<T, BLKV>), grid, dim3(256), 0, stream, (const T *)w, n,      \
                     packed, absmax, th)
  if (w_dtype == QL_BF16) {
    if (block == 128) QL_QUANT(uint16_t, 128); else QL_QUANT(uint16_t, 64);
  } else if (w_dtype == QL_F16) {
    if (block == 128) QL_QUANT(_Float16, 128); else QL_QUANT(_Float16, 64);
  } else {
    if (block == 128) QL_QUANT(float, 128); else QL_QUANT(float, 64);
  }
#undef QL_QUANT
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
  const int64_t nb2 = (nb + 255) / 256;  // one wave per DQ block, 4 per workgroup
  hipLaunchKernelGGL(k_dq_codes, dim3((unsigned)((nb2 + 3) / 4)), dim3(256), 0, stream, absmax, nb,
                     partial, np, q, sigma, mean_out);
  QL_HIP_CHECK_LAUNCH();
  return QL_OK;
}

int launch_nf4_dequantize(const uint8_t *packed, int64_t n, BlockScales sc, void *out,
                          int out_dtype, hipStream_t stream) {
  if (n <= 0) return QL_OK;
  // one wave per 4 x 64 x E elements (E = 8 for 16-bit, 4 for fp32 output)
  const int64_t per_wave = out_dtype == QL_F32 ? 1024 : 2048;
  const int64_t waves = (n + per_wave - 1) / per_wave;
  const dim3 grid((unsigned)((waves + 3) / 4));
  if (out_dtype == QL_BF16)
    hipLaunchKernelGGL(k_nf4_dequantize<uint16_t>, grid, dim3(256), 0, stream, packed, n, sc,
                       (uint16_t *)out);
  else if (out_dtype == QL_F16)
    hipLaunchKernelGGL(k_nf4_dequantize<_Float16>, grid, dim3(256), 0, stream, packed, n, sc,
                       (_Float16 *)out);
  else
    hipLaunchKernelGGL(k_nf4_dequantize<float>, grid, dim3(256), 0, stream, packed, n, sc,
                       (float *)out);
  QL_HIP_CHECK_LAUNCH();
  return QL_OK;
}

}  // namespace qlora
