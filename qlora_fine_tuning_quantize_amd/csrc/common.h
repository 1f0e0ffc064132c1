// common.h -- shared definitions of the gfx950 kernels of the QLoRA layer.
//
// Storage format (see include/qlora.h): row-major flattened weight, blocks
// of 64 (or 128) elements with one constant each, two 4-bit codebook indices
// per byte (element 2j in the high nibble).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "../../include/qlora.h"

namespace qlora {

// The 16 NF4 codepoints exactly as printed in the lookup table of
// "26. QLoRA and 4bit Quantization" (datawhalechina), Step 4, rounded to fp32.
#define QL_NF4_CODEBOOK_VALUES                                                       \
  {-1.0f,  -0.696f, -0.525f, -0.395f, -0.284f, -0.185f, -0.091f, 0.0f,              \
   0.080f, 0.161f,  0.246f,  0.338f,  0.441f,  0.563f,  0.723f,  1.0f}

// Decision thresholds of the nearest-codepoint search: t[i] separates
// codepoint i from codepoint i+1.  t[i] is the exact midpoint rounded down to
// fp32, so for any fp32 v:  v > t[i]  <=>  v is strictly nearer to cb[i+1]
// (an exact tie stays with the lower index).  Passed by value so the kernel
// reads them from scalar registers.
// Separate scalar fields (not an array) so the search below never turns
// into an indexed load from private memory.
struct NF4Thresholds {
  float t0, t1, t2, t3, t4, t5, t6, t7, t8, t9, t10, t11, t12, t13, t14;
};

// Host-side: thresholds derived from the codebook (defined in quant.hip).
NF4Thresholds nf4_thresholds();
const float *nf4_codebook_host();

// Device copy of the codebook (one per translation unit; read-only).
static __constant__ float c_nf4[16] = QL_NF4_CODEBOOK_VALUES;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two fp32 -> packed bf16x2 (low half = a), round to nearest even, as one
// v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const f32x2 f = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
}

__device__ __forceinline__ uint16_t f32_to_bf16_bits(float a) {
  return __builtin_bit_cast(uint16_t, (__bf16)a);
}

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// The two 16-bit formats of activations, outputs and matrix-core operands,
// named by their storage type: uint16_t holds bf16 bit patterns, _Float16
// IEEE binary16.  Conversions from fp32 round to nearest even (fp16
// overflows to infinity past its largest finite value, 65504).  The
// matrix-core ops multiply two operands of the format with fp32
// accumulation; operand layouts are the same for both formats.
template <typename H>
struct Half;

template <>
struct Half<uint16_t> {
  __device__ static __forceinline__ uint16_t bits(float a) { return f32_to_bf16_bits(a); }
  __device__ static __forceinline__ uint32_t pack2(float a, float b) { return pack_bf16x2(a, b); }
  // the value in the low / high half of a 32-bit word
  __device__ static __forceinline__ float lo(uint32_t w) { return __uint_as_float(w << 16); }
  __device__ static __forceinline__ float hi(uint32_t w) {
    return __uint_as_float(w & 0xFFFF0000u);
  }
  __device__ static __forceinline__ f32x16 mfma32(const u32x4 &a, const u32x4 &b,
                                                  const f32x16 &c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  __device__ static __forceinline__ f32x4 mfma16(const u32x4 &a, const u32x4 &b,
                                                 const f32x4 &c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
};

template <>
struct Half<_Float16> {
  __device__ static __forceinline__ uint16_t bits(float a) {
    return __builtin_bit_cast(uint16_t, (_Float16)a);
  }
  __device__ static __forceinline__ uint32_t pack2(float a, float b) {
    const f32x2 f = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, f16x2));
  }
  __device__ static __forceinline__ float lo(uint32_t w) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xFFFFu));
  }
  __device__ static __forceinline__ float hi(uint32_t w) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
  }
  __device__ static __forceinline__ f32x16 mfma32(const u32x4 &a, const u32x4 &b,
                                                  const f32x16 &c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  __device__ static __forceinline__ f32x4 mfma16(const u32x4 &a, const u32x4 &b,
                                                 const f32x4 &c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
};

template <typename T>
__device__ __forceinline__ float load_as_f32(const T *p, int64_t i);
template <>
__device__ __forceinline__ float load_as_f32<float>(const float *p, int64_t i) {
  return p[i];
}
template <>
__device__ __forceinline__ float load_as_f32<uint16_t>(const uint16_t *p, int64_t i) {
  return bf16_bits_to_f32(p[i]);
}
template <>
__device__ __forceinline__ float load_as_f32<_Float16>(const _Float16 *p, int64_t i) {
  return (float)p[i];
}

template <typename T>
__device__ __forceinline__ void store_from_f32(T *p, int64_t i, float v);
template <>
__device__ __forceinline__ void store_from_f32<float>(float *p, int64_t i, float v) {
  p[i] = v;
}
template <>
__device__ __forceinline__ void store_from_f32<uint16_t>(uint16_t *p, int64_t i, float v) {
  p[i] = f32_to_bf16_bits(v);
}
template <>
__device__ __forceinline__ void store_from_f32<_Float16>(_Float16 *p, int64_t i, float v) {
  p[i] = (_Float16)v;
}

// Host-side dispatch on a dtype: calls f with a null pointer of its storage
// type.  with_half: QL_F16 -> _Float16 *, otherwise uint16_t * (bf16);
// with_type: also QL_F32 -> float *.
template <typename F>
inline void with_half(int dtype, F &&f) {
  if (dtype == QL_F16) f((_Float16 *)nullptr);
  else f((uint16_t *)nullptr);
}
template <typename F>
inline void with_type(int dtype, F &&f) {
  if (dtype == QL_F32) f((float *)nullptr);
  else with_half(dtype, f);
}
// the storage type named by such a pointer
template <typename P>
using elem_of = typename std::remove_pointer<P>::type;

// The block constants of an NF4 weight: stored fp32 absmax, or rebuilt
// from their 8-bit codes with one rounding.  Kernels address them by the
// index c of a 64-element chunk of the flattened weight; an NF4 block is
// 64 << shift elements (64 or 128), so chunk c lies in block c >> shift.
struct BlockScales {
  const float *absmax;   // non-null: single-level form
  const int8_t *q;       // double-quantised form
  const float *sigma;
  const float *mu;
  int shift;             // 0: blocks of 64, 1: blocks of 128
  __device__ __forceinline__ int64_t index(int64_t c) const { return c >> shift; }
  __device__ __forceinline__ float operator()(int64_t c) const {
    const int64_t b = c >> shift;
    if (absmax) return absmax[b];
    return __builtin_fmaf((float)q[b], sigma[b >> 8], mu[0]);
  }
};

// LoRA dropout of the bypass input (the pages' LoraConfig lora_dropout):
// element e = m K + k of the activations [M, K] is kept when word e % 4 of
// Philox4x32-10 at counter (e / 4, 0, 0) under the 64-bit seed (k0 low
// word, k1 high) is >= thr = floor(p 2^32); kept inputs are scaled by
// 1/(1-p), which the kernels apply to the finished sums.
struct Dropout {
  uint32_t k0, k1, thr;
};

// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as
// easy as 1, 2, 3", SC'11) of counter (c0, c1, 0, 0) and key (k0, k1): ten
// rounds of two 32x32 -> 64-bit multiplies (0xD2511F53, 0xCD9E8D57) mixing
// the counter words with the key, the key advancing by the Weyl constants
// (0x9E3779B9, 0xBB67AE85) between rounds.
__device__ __forceinline__ u32x4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t k0,
                                               uint32_t k1) {
  uint32_t c2 = 0u, c3 = 0u;
#pragma unroll
  for (int round = 0; round < 10; ++round) {
    const uint32_t lo0 = 0xD2511F53u * c0, hi0 = __umulhi(0xD2511F53u, c0);
    const uint32_t lo1 = 0xCD9E8D57u * c2, hi1 = __umulhi(0xCD9E8D57u, c2);
    c0 = hi1 ^ c1 ^ k0;
    c1 = lo1;
    c2 = hi0 ^ c3 ^ k1;
    c3 = lo0;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return u32x4{c0, c1, c2, c3};
}

// keep bits of the 4 elements e .. e + 3 (e % 4 == 0): bit i for e + i
__device__ __forceinline__ uint32_t dropout_keep4(const Dropout &d, uint64_t e) {
  const uint64_t g = e >> 2;
  const u32x4 w = philox4x32_10((uint32_t)g, (uint32_t)(g >> 32), d.k0, d.k1);
  return (uint32_t)(w[0] >= d.thr) | ((uint32_t)(w[1] >= d.thr) << 1) |
         ((uint32_t)(w[2] >= d.thr) << 2) | ((uint32_t)(w[3] >= d.thr) << 3);
}

// keep bit of element e alone (the word e % 4 of its counter's draw)
__device__ __forceinline__ bool dropout_keep1(const Dropout &d, uint64_t e) {
  return (dropout_keep4(d, e) >> (e & 3u)) & 1u;
}

// 8 16-bit values (elements e .. e + 7 in order, e % 4 == 0) with the dropped
// ones set to zero
__device__ __forceinline__ u32x4 dropout_mask8(const Dropout &d, uint64_t e, u32x4 v) {
  const uint32_t bits = dropout_keep4(d, e) | (dropout_keep4(d, e + 4) << 4);
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const uint32_t lo = (bits >> (2 * w)) & 1u ? 0x0000FFFFu : 0u;
    const uint32_t hi = (bits >> (2 * w + 1)) & 1u ? 0xFFFF0000u : 0u;
    v[w] &= lo | hi;
  }
  return v;
}

}  // namespace qlora

#define QL_HIP_CHECK_LAUNCH()                               \
  do {                                                      \
    if (hipGetLastError() != hipSuccess) return QL_EHIP;    \
  } while (0)
