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

#include <algorithm>

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
// Quantisation proper.  Elements go in runs of 512 consecutive ones (8 NF4
// blocks of 64, or 4 of 128); in every run lane l takes the 8 elements
// 8l .. 8l + 7, so each block is held by a group of BLK / 8 lanes and every
// load and store instruction of the wave covers one contiguous span.  The
// group reduces |w| (DPP), then each lane finds its 8 indices and packs them
// into one 32-bit word.  The indices are those of the correctly rounded
// w / a: each lane takes a reciprocal of a once and the index of w times it;
// a lane with any element in a guard band (or with a block maximum outside
// the normal range) redoes its 8 elements with the division.
// ---------------------------------------------------------------------------

// The raw 16 bytes (16-bit types) or 32 bytes (fp32) of a lane's 8 elements.
template <typename T>
struct RunRaw {
  u32x4 v[sizeof(T) == 2 ? 1 : 2];
};

// Load the lane's 8 elements of the run starting at e0.  A run that is not
// whole loads from the start of the weight instead (n >= 8 there) and is
// reloaded element by element in quant_run; with n < 8 nothing is loaded.
// CHECKED = false promises e0 + 8 <= n (a straight load, no branch).
template <typename T, bool CHECKED = true>
__device__ __forceinline__ void load_run(const T *__restrict__ w, int64_t n, int64_t e0,
                                         RunRaw<T> &raw) {
  const int64_t ec = !CHECKED || e0 + 8 <= n ? e0 : 0;
  if (CHECKED && n < 8) {  // uniform: too short for any 8-element load
    for (int i = 0; i < (int)(sizeof(raw.v) / 16); ++i) raw.v[i] = u32x4{0u, 0u, 0u, 0u};
  } else {
#pragma unroll
    for (int i = 0; i < (int)(sizeof(raw.v) / 16); ++i)
      raw.v[i] = *reinterpret_cast<const u32x4 *>(reinterpret_cast<const uint8_t *>(w + ec) + 16 * i);
  }
}

template <typename T>
__device__ __forceinline__ void widen_run(const RunRaw<T> &raw, float (&v)[8]) {
  if constexpr (sizeof(T) == 2) {  // bf16 or fp16: widening is exact
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = Half<T>::lo(raw.v[0][i]);
      v[2 * i + 1] = Half<T>::hi(raw.v[0][i]);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = __uint_as_float(raw.v[i >> 2][i & 3]);
  }
}

// Code the lane's 8 values of a run: returns the packed word (element i in
// byte i / 2, high nibble for even i) and the group's block maximum in m.
// Wave-uniform call (the group reduction and the guard ballot span the wave).
template <int BLK>
__device__ __forceinline__ uint32_t code_run(const float (&v)[8], const BucketEntry *tab, int lane,
                                             float &m_out) {
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[i]));
  m = max_lanes<BLK / 8>(m);
  m_out = m;
  uint32_t word = 0x77777777u;  // a zero block: every element is the exact zero
  if (m != 0.0f) {
    bool slow = !(m >= 0x1p-125f && m <= 0x1p125f);
    if (!slow) {
      const float rm = __builtin_amdgcn_rcpf(m);
      uint64_t near = 0;
      word = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i)
        word |= nf4_index_fast(v[i] * rm, tab, near) << ((i & 1) ? 8 * (i >> 1) : 8 * (i >> 1) + 4);
      slow = (near >> lane) & 1u;
    }
    if (slow) {
      word = 0;
      for (int i = 0; i < 8; ++i)
        word |= nf4_index(v[i] / m, tab) << ((i & 1) ? 8 * (i >> 1) : 8 * (i >> 1) + 4);
    }
  }
  return word;
}

// Quantise the lane's 8 elements of the run at e0 (lane offset included),
// with bounds checks: writes the packed word and, from the first lane of each
// group, the block constant.  Returns the block maximum (0 past the end).
template <typename T, int BLK>
__device__ __forceinline__ float quant_run(const T *__restrict__ w, int64_t n, int64_t e0,
                                           float (&v)[8], const BucketEntry *tab, int lane,
                                           uint8_t *__restrict__ packed,
                                           float *__restrict__ absmax) {
  if (e0 + 8 > n) {  // the ragged end (or past it): elements past n count as 0
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = (e0 + i < n) ? load_as_f32(w, e0 + i) : 0.0f;
  }
  float m;
  uint32_t word = code_run<BLK>(v, tab, lane, m);
  if (e0 >= n) return 0.0f;  // lanes past the end only helped the group reduction
  if (e0 + 8 <= n) {
    *reinterpret_cast<uint32_t *>(packed + (e0 >> 1)) = word;
  } else {
    // nibbles of elements past n are 0
    for (int i = 0; i < 8; ++i)
      if (e0 + i >= n) word &= ~(0xFu << ((i & 1) ? 8 * (i >> 1) : 8 * (i >> 1) + 4));
    for (int b = 0; b < 4; ++b)
      if (e0 + 2 * b < n) packed[(e0 >> 1) + b] = (uint8_t)(word >> (8 * b));
  }
  if ((lane & (BLK / 8 - 1)) == 0) absmax[e0 / BLK] = m;
  return m;
}

// Single-level form, one workgroup of 256 threads (number wg of its weight):
// a wave owns 2 runs; all loads are issued first.
template <typename T, int BLK>
__device__ __forceinline__ void quantize_wg(const T *__restrict__ w, int64_t n,
                                            uint8_t *__restrict__ packed,
                                            float *__restrict__ absmax, const NF4Thresholds &th,
                                            BucketEntry *tab, int64_t wg) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = wg * 4 + (threadIdx.x >> 6);
  constexpr int R = 2;
  RunRaw<T> raw[R];
#pragma unroll
  for (int j = 0; j < R; ++j) load_run(w, n, wave * (R * 512) + j * 512 + lane * 8, raw[j]);
  build_buckets(tab, th, threadIdx.x);
  __syncthreads();
#pragma unroll
  for (int j = 0; j < R; ++j) {
    float v[8];
    widen_run(raw[j], v);
    quant_run<T, BLK>(w, n, wave * (R * 512) + j * 512 + lane * 8, v, tab, lane, packed, absmax);
  }
}

template <typename T, int BLK>
__global__ __launch_bounds__(256) void k_nf4_quantize(const T *__restrict__ w, int64_t n,
                                                      uint8_t *__restrict__ packed,
                                                      float *__restrict__ absmax,
                                                      NF4Thresholds th) {
  __shared__ BucketEntry tab[kBuckets];
  quantize_wg<T, BLK>(w, n, packed, absmax, th, tab, blockIdx.x);
}

// ---------------------------------------------------------------------------
// Double-quantised form, pass 1: the quantisation above, plus the exact sum
// of the block constants (Gemma lesson 09, sec. 9.2.2 centres the constants
// on their mean).  A block constant a >= 0 is an integer multiple of 2^-149:
// a = M 2^(e-1) 2^-149 with M its 24-bit significand (hidden bit included)
// and e its biased exponent (e = 1 for subnormals, M then without the hidden
// bit), so a 2^149 < 2^277.  The workgroup adds M 2^(e-1) into ten 32-bit
// digit positions kept as 64-bit counters in LDS (integer atomics: the result
// does not depend on their order), so the sum is exact whatever the range of
// the constants; an infinite constant is counted apart.  Each workgroup
// writes its counters as one partial sum (digit-major: partial[d * grid +
// workgroup]).  The workgroups walk the runs in a grid-stride loop (grid
// capped at kQdMaxGroups, so the partials stay few), kQdRuns runs per wave
// per step.
// ---------------------------------------------------------------------------
constexpr int kQdThreads = 1024;
constexpr int kQdRuns = 2;  // runs of 512 elements per wave and step

// v 2^sh (in units of 2^-149) into the digit counters; v < 2^64, sh <= 253.
__device__ __forceinline__ void add_shifted(unsigned long long *dig, uint64_t v, int sh) {
  const int d = sh >> 5, o = sh & 31;
  const uint64_t lo = v << o;                 // low 64 bits of v 2^o
  const uint64_t hi = o ? v >> (64 - o) : 0;  // the bits above them (< 2^31)
  atomicAdd(&dig[d], lo & 0xFFFFFFFFull);
  if (lo >> 32) atomicAdd(&dig[d + 1], lo >> 32);
  if (hi) atomicAdd(&dig[d + 2], hi);
}

// A lane's running sum of the constants it owns, acc 2^base: a constant
// M 2^sh with base <= sh <= base + 24 adds M << (sh - base) (< 2^48) to acc,
// which is moved into the digits before it could reach 2^63; the first
// constant sets base = sh - 8 (so constants 2^8 times smaller still fit),
// and constants outside the window go to the digits directly.  The
// constants of one weight rarely span more than a few binades, so the digits
// (LDS atomics) are touched about once per lane.
struct LaneSum {
  uint64_t acc;
  int base;
};

__device__ __forceinline__ void lane_add(LaneSum &S, float m, unsigned long long *dig) {
  const uint32_t u = __float_as_uint(m);
  const uint32_t e = u >> 23;  // m >= 0: no sign bit
  if (e == 255u) {
    atomicAdd(&dig[kQdInfDigit], 1ull);
    return;
  }
  const uint64_t M = e ? ((u & 0x7FFFFFu) | 0x800000u) : (u & 0x7FFFFFu);
  if (M == 0) return;
  const int sh = e ? (int)e - 1 : 0;  // m 2^149 = M 2^sh, sh <= 253
  if (S.base < 0) S.base = sh > 8 ? sh - 8 : 0;
  const int k = sh - S.base;
  if (k < 0 || k > 24) {
    add_shifted(dig, M, sh);
    return;
  }
  if (S.acc >> 62) {
    add_shifted(dig, S.acc, S.base);
    S.acc = 0;
  }
  S.acc += M << k;
}

// One workgroup (number wg of `groups` on this weight; tab and dig in LDS).
template <typename T, int BLK>
__device__ __forceinline__ void quantize_dq_wg(const T *__restrict__ w, int64_t n,
                                               uint8_t *__restrict__ packed,
                                               float *__restrict__ absmax, const NF4Thresholds &th,
                                               unsigned long long *__restrict__ partial,
                                               BucketEntry *tab, unsigned long long *dig, int wg,
                                               int groups) {
  const int lane = threadIdx.x & 63;
  constexpr int WPG = kQdThreads / 64;
  constexpr int R = kQdRuns;
  const int64_t step = (int64_t)groups * WPG;
  const int64_t full = n / (R * 512);  // steps wholly inside the weight
  // the wave's step index, wave-uniform (scalar) for the address math
  int64_t c = (int64_t)wg * WPG + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  build_buckets(tab, th, threadIdx.x);
  if (threadIdx.x < kQdDigits) dig[threadIdx.x] = 0;
  __syncthreads();
  LaneSum lsum{0ull, -1};
  RunRaw<T> raw[R];
  // Whole steps: all R loads of a step are issued together, then the step is
  // coded and stored.  (Loads and stores share one completion counter, so a
  // load issued ahead of a step's stores would be waited for together with
  // them: the overlap of memory and coding comes from the other waves of the
  // CU instead.)
  for (; c < full; c += step) {
#pragma unroll
    for (int j = 0; j < R; ++j) load_run<T, false>(w, n, c * (R * 512) + j * 512 + lane * 8, raw[j]);
    uint32_t *pk = reinterpret_cast<uint32_t *>(packed + c * (R * 256)) + lane;
    float *am = absmax + c * (R * 512 / BLK) + lane / (BLK / 8);
#pragma unroll
    for (int j = 0; j < R; ++j) {
      float v[8], m;
      widen_run(raw[j], v);
      pk[j * 64] = code_run<BLK>(v, tab, lane, m);
      am[j * (512 / BLK)] = m;  // every lane of the group stores the same m
      if ((lane & (BLK / 8 - 1)) == 0) lane_add(lsum, m, dig);
    }
  }
  if (c * (R * 512) < n) {  // the ragged last step (c == full), wave-uniform
#pragma unroll
    for (int j = 0; j < R; ++j) {
      const int64_t e0 = c * (R * 512) + j * 512 + lane * 8;
      load_run(w, n, e0, raw[j]);
      float v[8];
      widen_run(raw[j], v);
      const float m = quant_run<T, BLK>(w, n, e0, v, tab, lane, packed, absmax);
      if ((lane & (BLK / 8 - 1)) == 0 && e0 < n) lane_add(lsum, m, dig);
    }
  }
  if (lsum.acc) add_shifted(dig, lsum.acc, lsum.base);
  __syncthreads();
  // digit-major: partial[d * groups + wg]
  if (threadIdx.x < kQdDigits) partial[(int64_t)threadIdx.x * groups + wg] = dig[threadIdx.x];
}

template <typename T, int BLK>
__global__ __launch_bounds__(kQdThreads, 8) void k_nf4_quantize_dq(const T *__restrict__ w, int64_t n,
                                                                uint8_t *__restrict__ packed,
                                                                float *__restrict__ absmax,
                                                                NF4Thresholds th,
                                                                unsigned long long *__restrict__ partial) {
  __shared__ BucketEntry tab[kBuckets];
  __shared__ unsigned long long dig[kQdDigits];
  quantize_dq_wg<T, BLK>(w, n, packed, absmax, th, partial, tab, dig, blockIdx.x, gridDim.x);
}


// ---------------------------------------------------------------------------
// Double-quantised form, pass 2: every workgroup (16 waves) first adds the
// partial sums digit by digit (64-bit integers: exact), carries them into
// 32-bit limbs and rounds the exact sum S once to fp64 (nearest, ties to
// even); mu = fp32(fp64(S) / nb), the fp64 division correctly rounded.  Then
// each wave takes DQ blocks of 256 constants (4 per lane) in a grid-stride
// loop: d = a - mu, sigma = max|d| / 127, code = clamp(rint(d / sigma),
// +-127).  The first block's constants are loaded before the sum.
// ---------------------------------------------------------------------------

// 64-bit wave sum (shuffles; the value of every lane is the sum).
__device__ __forceinline__ unsigned long long wave_sum_u64(unsigned long long v) {
#pragma unroll
  for (int delta = 32; delta > 0; delta >>= 1) v += __shfl_xor(v, delta, 64);
  return v;
}

// L[i] of a 10-limb array held in registers (0 past the end).
__device__ __forceinline__ uint32_t limb(const uint32_t (&L)[10], int i) {
  uint32_t r = 0;
#pragma unroll
  for (int k = 0; k < 10; ++k) r = k == i ? L[k] : r;
  return r;
}

// Bits [lo, lo + 64) of the little-endian limbs L.
__device__ __forceinline__ uint64_t limb_bits(const uint32_t (&L)[10], int lo) {
  const int w = lo >> 5, o = lo & 31;
  const uint64_t low = (uint64_t)limb(L, w) | ((uint64_t)limb(L, w + 1) << 32);
  const uint64_t high = limb(L, w + 2);
  return o ? (low >> o) | (high << (64 - o)) : low;
}

// mu from the digit totals (one thread; the limbs stay in registers).
__device__ float exact_mean(const unsigned long long *tot, int64_t nb) {
  if (tot[kQdInfDigit] != 0) return __builtin_huge_valf();
  uint32_t L[10];
  uint64_t carry = 0;
#pragma unroll
  for (int k = 0; k < 10; ++k) {
    const uint64_t t = tot[k] + carry;  // tot[k] < 2^64 - 2^32, carry < 2^32
    L[k] = (uint32_t)t;
    carry = t >> 32;
  }
  // S < 2^317: the carry out of limb 9 is 0
  int top = -1;
#pragma unroll
  for (int k = 0; k < 10; ++k) top = L[k] ? k : top;
  double sum = 0.0;
  if (top >= 0) {
    int p = 32 * top + 31 - __builtin_clz(limb(L, top));  // leading bit of S
    if (p < 53) {
      sum = ldexp((double)limb_bits(L, 0), -149);  // exact
    } else {
      uint64_t m = limb_bits(L, p - 52) & ((1ull << 53) - 1);
      const int rp = p - 53;  // round bit
      const uint32_t lr = limb(L, rp >> 5);
      const bool round = (lr >> (rp & 31)) & 1u;
      bool sticky = (lr & ((1u << (rp & 31)) - 1u)) != 0;
#pragma unroll
      for (int k = 0; k < 10; ++k) sticky |= k < (rp >> 5) && L[k] != 0;
      if (round && (sticky || (m & 1))) {
        ++m;
        if (m >> 53) {
          m >>= 1;
          ++p;
        }
      }
      sum = ldexp((double)m, p - 52 - 149);
    }
  }
  return (float)(sum / (double)nb);
}

constexpr int kDcThreads = 1024;
static_assert(kDcThreads / 64 >= kQdDigits, "one wave per digit counter");
static_assert(kQdMaxGroups % 64 == 0, "whole partials per lane");

// One workgroup (number wg of `groups` on this weight; tot and s_mu in LDS).
__device__ __forceinline__ void dq_codes_wg(const float *__restrict__ a, int64_t nb,
                                            const unsigned long long *__restrict__ partial,
                                            int n_partial, int8_t *__restrict__ q,
                                            float *__restrict__ sigma, float *__restrict__ mean_out,
                                            unsigned long long *tot, float *s_mu, int wg,
                                            int groups) {
  constexpr int WPG = kDcThreads / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t nb2 = (nb + 255) / 256;
  const int64_t step = (int64_t)groups * WPG;
  int64_t b2 = (int64_t)wg * WPG + wave;
  auto load4 = [&](int64_t blk, float (&av)[4]) {
    const int64_t j0 = blk * 256 + 4 * lane;
    if (j0 + 4 <= nb) {
      const f32x4 t = *reinterpret_cast<const f32x4 *>(a + j0);
      av[0] = t[0]; av[1] = t[1]; av[2] = t[2]; av[3] = t[3];
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) av[i] = j0 + i < nb ? a[j0 + i] : 0.0f;
    }
  };
  float av[4];
  load4(b2 < nb2 ? b2 : 0, av);

  // wave k < kQdDigits adds digit k of every partial (lane l takes partials
  // l, l + 64, ...; n_partial <= kQdMaxGroups), then one wave-wide sum;
  // thread 0 rounds the totals
  if (wave < kQdDigits) {
    // at most kQdMaxGroups / 64 partials per lane, all loads in flight at once
    unsigned long long pk[kQdMaxGroups / 64];
#pragma unroll
    for (int i = 0; i < kQdMaxGroups / 64; ++i) {
      const int p = lane + 64 * i;
      pk[i] = p < n_partial ? partial[(int64_t)wave * n_partial + p] : 0ull;
    }
    unsigned long long dk = 0;
#pragma unroll
    for (int i = 0; i < kQdMaxGroups / 64; ++i) dk += pk[i];
    dk = wave_sum_u64(dk);
    if (lane == 0) tot[wave] = dk;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    *s_mu = exact_mean(tot, nb);
    if (wg == 0) mean_out[0] = *s_mu;
  }
  __syncthreads();
  const float mu = *s_mu;

  for (; b2 < nb2; b2 += step) {
    const int64_t j0 = b2 * 256 + 4 * lane;
    float d4[4], amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      d4[i] = j0 + i < nb ? av[i] - mu : 0.0f;
      amax = fmaxf(amax, fabsf(d4[i]));
    }
    if (b2 + step < nb2) load4(b2 + step, av);  // wave-uniform
#pragma unroll
    for (int delta = 32; delta > 0; delta >>= 1) amax = fmaxf(amax, __shfl_xor(amax, delta, 64));
    const float sg = amax / 127.0f;
    uint32_t word = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float c = 0.0f;
      if (sg != 0.0f) {
        c = __builtin_rintf(d4[i] / sg);
        c = fminf(fmaxf(c, -127.0f), 127.0f);
      }
      word |= ((uint32_t)(int)c & 0xFFu) << (8 * i);
    }
    if (j0 + 4 <= nb && ((uintptr_t)q & 3u) == 0) {
      *reinterpret_cast<uint32_t *>(q + j0) = word;
    } else {  // ragged end, or a code array without 4-byte alignment
      for (int i = 0; i < 4; ++i)
        if (j0 + i < nb) q[j0 + i] = (int8_t)(word >> (8 * i));
    }
    if (lane == 0) sigma[b2] = sg;
  }
}

__global__ __launch_bounds__(kDcThreads) void k_dq_codes(const float *__restrict__ a, int64_t nb,
                                                         const unsigned long long *__restrict__ partial,
                                                         int n_partial, int8_t *__restrict__ q,
                                                         float *__restrict__ sigma,
                                                         float *__restrict__ mean_out) {
  __shared__ unsigned long long tot[kQdDigits];
  __shared__ float s_mu;
  dq_codes_wg(a, nb, partial, n_partial, q, sigma, mean_out, tot, &s_mu, blockIdx.x, gridDim.x);
}

// ---------------------------------------------------------------------------
// Several weights per launch (a model's tensors quantised together when it
// is loaded).  Workgroups [f[t], f[t + 1]) run weight t exactly as its own
// launch would (the same workgroup count, numbering and partial layout), so
// the results are those of one launch per weight; small weights no longer
// pay a launch each, and their workgroups fill the chip beside the large
// ones.  At most kQmMax weights per launch.
// ---------------------------------------------------------------------------
struct QuantBatch {
  const void *w[kQmMax];
  int64_t n[kQmMax];
  uint8_t *packed[kQmMax];
  float *absmax[kQmMax];
  unsigned long long *partial[kQmMax];
  int8_t *q[kQmMax];
  float *sigma[kQmMax];
  float *mean[kQmMax];
  int g0[kQmMax + 1];  // first workgroup of each weight, quantisation launch
  int h0[kQmMax + 1];  // first workgroup of each weight, codes launch
  int count;
};

// Entry t of a kernel-argument array for a workgroup-uniform t: selects over
// constant indices, so the array stays in scalar registers and is never
// indexed in memory.
template <typename P, int N>
__device__ __forceinline__ P pick(const P (&a)[N], int t) {
  P r = a[0];
#pragma unroll
  for (int i = 1; i < N; ++i) r = i == t ? a[i] : r;
  return r;
}

// The weight that workgroup wg works on, from the first-workgroup offsets f.
__device__ __forceinline__ int batch_member(const int (&f)[kQmMax + 1], int count, int wg) {
  int t = 0;
#pragma unroll
  for (int i = 1; i < kQmMax; ++i) t += (i < count && wg >= f[i]) ? 1 : 0;
  return t;
}

template <typename T, int BLK>
__global__ __launch_bounds__(256) void k_nf4_quantize_many(QuantBatch b, NF4Thresholds th) {
  __shared__ BucketEntry tab[kBuckets];
  const int t = batch_member(b.g0, b.count, blockIdx.x);
  quantize_wg<T, BLK>((const T *)pick(b.w, t), pick(b.n, t), pick(b.packed, t),
                      pick(b.absmax, t), th, tab, (int64_t)blockIdx.x - pick(b.g0, t));
}

template <typename T, int BLK>
__global__ __launch_bounds__(kQdThreads, 8) void k_nf4_quantize_dq_many(QuantBatch b,
                                                                     NF4Thresholds th) {
  __shared__ BucketEntry tab[kBuckets];
  __shared__ unsigned long long dig[kQdDigits];
  const int t = batch_member(b.g0, b.count, blockIdx.x);
  const int f = pick(b.g0, t);
  quantize_dq_wg<T, BLK>((const T *)pick(b.w, t), pick(b.n, t), pick(b.packed, t),
                         pick(b.absmax, t), th, pick(b.partial, t), tab, dig,
                         (int)blockIdx.x - f, pick(b.g0, t + 1) - f);
}

__global__ __launch_bounds__(kDcThreads) void k_dq_codes_many(QuantBatch b, int block) {
  __shared__ unsigned long long tot[kQdDigits];
  __shared__ float s_mu;
  const int t = batch_member(b.h0, b.count, blockIdx.x);
  const int f = pick(b.h0, t);
  const int64_t nb = (pick(b.n, t) + block - 1) / block;
  dq_codes_wg(pick(b.absmax, t), nb, pick(b.partial, t), pick(b.g0, t + 1) - pick(b.g0, t),
              pick(b.q, t), pick(b.sigma, t), pick(b.mean, t), tot, &s_mu, (int)blockIdx.x - f,
              pick(b.h0, t + 1) - f);
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
// Workgroups of one weight's launch: single-level quantisation (one wave per
// 1024 elements, 4 waves per workgroup), the double-quantised form (a
// grid-stride loop over steps of 16 waves x 1024 elements, at most
// kQdMaxGroups workgroups) and its codes (16 DQ blocks per workgroup and
// step, at most 256 workgroups).
static int64_t quant_groups(int64_t n) { return ((n + 1023) / 1024 + 3) / 4; }
static int quant_dq_groups(int64_t n) {
  const int64_t chunks = (n + kQdRuns * 512 - 1) / (kQdRuns * 512);
  return (int)std::min<int64_t>(kQdMaxGroups, (chunks + kQdThreads / 64 - 1) / (kQdThreads / 64));
}
static int dq_code_groups(int64_t nb) {
  const int64_t nb2 = (nb + 255) / 256;
  return (int)std::min<int64_t>(256, (nb2 + 15) / 16);
}

int launch_nf4_quantize(const void *w, int w_dtype, int64_t n, int block, uint8_t *packed,
                        float *absmax, hipStream_t stream) {
  if (n <= 0) return QL_OK;
  const dim3 grid((unsigned)quant_groups(n));
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

int launch_nf4_quantize_dq(const void *w, int w_dtype, int64_t n, int block, uint8_t *packed,
                           float *absmax, unsigned long long *partial, int8_t *q, float *sigma,
                           float *mean_out, hipStream_t stream) {
  if (n <= 0) return QL_OK;
  const int64_t nb = (n + block - 1) / block;
  if (nb >= (int64_t(1) << 31)) return QL_EUNSUPPORTED;  // keeps the 64-bit digit sums exact
  const int groups = quant_dq_groups(n);
  const NF4Thresholds th = nf4_thresholds();
#define QL_QUANT(T, BLKV)                                                                        \
  hipLaunchKernelGGL((k_nf4_quantize_dq<T, BLKV>), dim3(groups), dim3(kQdThreads), 0, stream,     \
                     (const T *)w, n, packed, absmax, th, partial)
  if (w_dtype == QL_BF16) {
    if (block == 128) QL_QUANT(uint16_t, 128); else QL_QUANT(uint16_t, 64);
  } else if (w_dtype == QL_F16) {
    if (block == 128) QL_QUANT(_Float16, 128); else QL_QUANT(_Float16, 64);
  } else {
    if (block == 128) QL_QUANT(float, 128); else QL_QUANT(float, 64);
  }
#undef QL_QUANT
  QL_HIP_CHECK_LAUNCH();
  hipLaunchKernelGGL(k_dq_codes, dim3(dq_code_groups(nb)), dim3(kDcThreads), 0, stream, absmax, nb,
                     partial, groups, q, sigma, mean_out);
  QL_HIP_CHECK_LAUNCH();
  return QL_OK;
}

int launch_nf4_quantize_many(int count, const void *const *w, int w_dtype, const int64_t *n,
                             int block, bool dq, uint8_t *const *packed, float *const *absmax,
                             unsigned long long *const *partial, int8_t *const *q,
                             float *const *sigma, float *const *mean, hipStream_t stream) {
  if (count <= 0) return QL_OK;
  if (count > kQmMax) return QL_EINVAL;
  const NF4Thresholds th = nf4_thresholds();
  // a launch stays below 2^31 work-items: weights past that go to another one
  const int64_t cap = (int64_t(1) << 31) / (dq ? kQdThreads : 256);
  for (int i0 = 0; i0 < count;) {
    QuantBatch b{};
    int64_t g = 0;
    int h = 0, j = 0;
    for (; i0 + j < count && j < kQmMax; ++j) {
      const int i = i0 + j;
      const int64_t gi = dq ? quant_dq_groups(n[i]) : quant_groups(n[i]);
      if (j > 0 && g + gi > cap) break;
      b.w[j] = w[i];
      b.n[j] = n[i];
      b.packed[j] = packed[i];
      b.absmax[j] = absmax[i];
      b.g0[j] = (int)g;
      b.h0[j] = h;
      if (dq) {
        b.partial[j] = partial[i];
        b.q[j] = q[i];
        b.sigma[j] = sigma[i];
        b.mean[j] = mean[i];
        h += dq_code_groups((n[i] + block - 1) / block);
      }
      g += gi;
    }
    b.count = j;
    for (int k = j; k <= kQmMax; ++k) {
      b.g0[k] = (int)g;
      b.h0[k] = h;
    }
#define QL_QUANT(T, BLKV)                                                                         \
  if (dq)                                                                                          \
    hipLaunchKernelGGL((k_nf4_quantize_dq_many<T, BLKV>), dim3((unsigned)g), dim3(kQdThreads), 0, \
                       stream, b, th);                                                             \
  else                                                                                             \
    hipLaunchKernelGGL((k_nf4_quantize_many<T, BLKV>), dim3((unsigned)g), dim3(256), 0, stream, b, \
                       th)
    if (w_dtype == QL_BF16) {
      if (block == 128) QL_QUANT(uint16_t, 128); else QL_QUANT(uint16_t, 64);
    } else if (w_dtype == QL_F16) {
      if (block == 128) QL_QUANT(_Float16, 128); else QL_QUANT(_Float16, 64);
    } else {
      if (block == 128) QL_QUANT(float, 128); else QL_QUANT(float, 64);
    }
#undef QL_QUANT
    QL_HIP_CHECK_LAUNCH();
    if (dq) {
      hipLaunchKernelGGL(k_dq_codes_many, dim3((unsigned)h), dim3(kDcThreads), 0, stream, b, block);
      QL_HIP_CHECK_LAUNCH();
    }
    i0 += j;
  }
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
