// Device-side helpers shared by the Conv3D kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace conv3d {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// fp32 -> bf16, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint16_t f2bf(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }
__device__ __forceinline__ float bf2f(uint16_t b) { return __builtin_bit_cast(float, (unsigned)b << 16); }
// B(x): round an fp32 value to bf16 and back.
__device__ __forceinline__ float rbf(float f) { return bf2f(f2bf(f)); }
// Two fp32 values as bf16 (lo in the low half), one v_cvt_pk_bf16_f32.
__device__ __forceinline__ unsigned pack2(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(unsigned, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t));
}
__device__ __forceinline__ float lane_bf(const u32x4_t& v, int e) {
  return bf2f((uint16_t)(v[e >> 1] >> (16 * (e & 1))));
}

}  // namespace conv3d
