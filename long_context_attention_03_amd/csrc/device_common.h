// device_common.h -- gfx950 device helpers shared by the library's kernels (not by the oracle).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace csah {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float u2f(uint32_t u) { return __uint_as_float(u); }
__device__ __forceinline__ uint32_t f2u(float f) { return __float_as_uint(f); }

// 2^(e-127) for an E8M0 byte, as binary32 (e = 0 is the subnormal 2^-127, 255 is NaN).
__device__ __forceinline__ float e8m0_to_f32(uint32_t e) {
  e &= 255u;
  uint32_t bits = e == 0 ? 0x00400000u : (e == 255 ? 0x7FC00000u : (e << 23));
  return u2f(bits);
}

// Two E2M1 elements of byte `sel` (low nibble first) as fp32, unscaled.
template <int SEL>
__device__ __forceinline__ f32x2 fp4x2_to_f32(uint32_t word) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, SEL);
}

// Monotone map of binary32 onto uint32 (larger float -> larger key); -0 must be folded first.
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = f2u(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_to_float(uint32_t k) {
  return u2f((k & 0x80000000u) ? (k ^ 0x80000000u) : ~k);
}

// Butterfly add across lanes lane ^ 1 and lane ^ 2 (DPP quad permutes).
// Every lane reads a lane of its own quad, so bound_ctrl never applies; setting it lets the
// compiler fold the move into the add (one DPP add instead of a DPP move and an add).
__device__ __forceinline__ float quad_xor1_add(float v) {
  int t = __builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, true);  // [1,0,3,2]
  return v + __int_as_float(t);
}
__device__ __forceinline__ float quad_xor2_add(float v) {
  int t = __builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, true);  // [2,3,0,1]
  return v + __int_as_float(t);
}

__device__ __forceinline__ float shfl_xor_f(float v, int o) { return __shfl_xor(v, o, 64); }

// 64-bit lane mask of lanes whose predicate holds.
__device__ __forceinline__ uint64_t ballot64(bool p) { return __ballot(p); }

// ---- encoders used by the compressor (independent of any host code) ------------------------

// binary32 -> OCP E4M3 (bias 7, max 448), round to nearest even, saturating; NaN -> 0x7F.
__device__ __forceinline__ uint32_t f32_to_e4m3(float f) {
  uint32_t u = f2u(f);
  uint32_t sign = (u >> 24) & 0x80u;
  float a = fabsf(f);
  if (!(a == a)) return 0x7Fu;
  if (a >= 464.0f) return sign | 0x7Eu;        // at or above the midpoint to 512: saturate
  if (a < 0.015625f) {                         // below 2^-6: subnormal grid of step 2^-9
    uint32_t q = (uint32_t)__builtin_rintf(a * 512.0f);  // 0..8; 8 is the smallest normal
    return sign | q;
  }
  uint32_t ua = f2u(a);
  uint32_t r = (ua + 0x7FFFFu + ((ua >> 20) & 1u)) >> 20;  // keep 3 mantissa bits, ties to even
  uint32_t code = r - ((127u - 7u) << 3);
  if (code > 0x7Eu) code = 0x7Eu;
  return sign | code;
}

// E2M1 code of a value already divided by its block scale; ties to even, saturating at 6.
__device__ __forceinline__ uint32_t f32_to_e2m1(float r) {
  uint32_t sign = (f2u(r) >> 28) & 0x8u;
  float a = fabsf(r);
  uint32_t code;
  if (a < 2.0f) {
    code = (uint32_t)__builtin_rintf(a * 2.0f);           // 0,0.5,1,1.5,2 -> codes 0..4
  } else if (a < 4.0f) {
    code = (uint32_t)__builtin_rintf(a) + 2u;              // 2,3,4 -> codes 4,5,6
  } else {
    float q = __builtin_rintf(a * 0.5f);                   // 4,6,8 -> 2,3,4
    code = q >= 3.0f ? 7u : 6u;                            // 8 saturates to 6
  }
  return sign | code;
}

// RoPE angle of rotary pair j (of R/2) at position p, as (cos, sin) in fp64: RoFormer's general
// form turns pair j by p * base^(-2j/R); the inverse turns it back. fp64 keeps the angle exact
// enough at positions of 2^20 and beyond (fp32 would lose the angle to within 0.1 radian).
__device__ __forceinline__ void rope_cos_sin(double p, int j, int R, double base, bool inverse,
                                             double& c, double& s) {
  double ang = p * pow(base, -2.0 * j / R);
  if (inverse) ang = -ang;
  sincos(ang, &s, &c);
}

}  // namespace csah
