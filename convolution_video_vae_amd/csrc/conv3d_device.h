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

// The fused post-operations after the row norm, for one value v of a pixel
// whose channel row has norm den = max(sqrt(sum v^2), 1e-12), passed as
// rden = 1 / den (correctly rounded, once per pixel):
//   nrm = B(v / den), scl = B(nrm * sqrt(C)), aff = B(scl * gamma),
//   out = B(aff / (1 + e^-aff)).
// v / den is formed as v * rden (within 1.5 fp32 ulps of the quotient). e^x
// is 2^(x log2 e) with the product split into a rounded part t and its
// remainder r (from an fma and the low half of log2 e), so the hardware
// exp2 of t times 1 + r ln 2 keeps the result within about 2 ulps for any
// |x| of a normalised row; the quotient is aff times the hardware
// reciprocal. Each stays a few fp32 ulps from the exact value, far below the
// bf16 rounding that follows, and the three kernels that finish the contract
// share this code, so they agree bit for bit.
// aff / (1 + e^-aff) in fp32, before its final rounding.
__device__ __forceinline__ float silu_f32(float aff) {
  constexpr float kLog2eHi = 1.44269502162933349609375f;   // fp32 nearest log2(e)
  constexpr float kLog2eLo = 1.925963033500011e-08f;       // log2(e) - kLog2eHi
  constexpr float kLn2 = 0.693147182464599609375f;
  const float x = -aff;
  const float t = x * kLog2eHi;
  const float r = __builtin_fmaf(x, kLog2eLo, __builtin_fmaf(x, kLog2eHi, -t));
  const float e2 = __builtin_amdgcn_exp2f(t);
  const float ex = __builtin_fmaf(e2, r * kLn2, e2);
  return aff * __builtin_amdgcn_rcpf(1.0f + ex);
}
__device__ __forceinline__ float norm_silu_value(float v, float rden, float sqrt_c, float g) {
  const float nrm = rbf(v * rden);
  const float scl = rbf(nrm * sqrt_c);
  const float aff = rbf(scl * g);
  return rbf(silu_f32(aff));
}

// The low and high bf16 halves of a packed pair as fp32 (one shift / mask).
__device__ __forceinline__ float bf_lo(unsigned u) { return __builtin_bit_cast(float, u << 16); }
__device__ __forceinline__ float bf_hi(unsigned u) { return __builtin_bit_cast(float, u & 0xffff0000u); }

// norm_silu_value on both halves of a packed pair of values v with their
// gammas g, as a packed pair: the same operations and roundings, two values
// per conversion.
__device__ __forceinline__ unsigned norm_silu_pair(unsigned v, unsigned g, float rden,
                                                   float sqrt_c) {
  const unsigned nrm = pack2(bf_lo(v) * rden, bf_hi(v) * rden);
  const unsigned scl = pack2(bf_lo(nrm) * sqrt_c, bf_hi(nrm) * sqrt_c);
  const unsigned aff = pack2(bf_lo(scl) * bf_lo(g), bf_hi(scl) * bf_hi(g));
  return pack2(silu_f32(bf_lo(aff)), silu_f32(bf_hi(aff)));
}

}  // namespace conv3d
