// common.h -- shared definitions of the gfx950 kernels of the QLoRA layer.
//
// Storage format (see include/qlora.h): row-major flattened weight, blocks
// of 64 elements with one constant each, two 4-bit codebook indices per byte
// (element 2j in the high nibble).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

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

// The constant of NF4 block b: stored fp32 absmax, or rebuilt from its 8-bit
// code with one rounding.
struct BlockScales {
  const float *absmax;   // non-null: single-level form
  const int8_t *q;       // double-quantised form
  const float *sigma;
  const float *mu;
  __device__ __forceinline__ float operator()(int64_t b) const {
    if (absmax) return absmax[b];
    return __builtin_fmaf((float)q[b], sigma[b >> 8], mu[0]);
  }
};

}  // namespace qlora

#define QL_HIP_CHECK_LAUNCH()                               \
  do {                                                      \
    if (hipGetLastError() != hipSuccess) return QL_EHIP;    \
  } while (0)
