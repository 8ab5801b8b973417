// Device helpers shared by the gfx950 kernels of libsvdq.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace svdq {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef uint32_t u32;

// ---- bit-level number formats (device side) --------------------------------
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) {
  return __uint_as_float(h << 16);
}

// Round-to-nearest-even fp32 -> bf16 bits (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// Two fp32 -> packed bf16 pair (a in the low half) with the hardware
// conversion v_cvt_pk_bf16_f32: round to nearest even, the same bits as
// f32_to_bf16_bits for every finite input.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef __bf16 bf2_t __attribute__((ext_vector_type(2)));
  typedef float f2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2_t{a, b}), bf2_t));
}

// fp32 (finite, >= 0) -> fp16 bits, round-to-nearest-even, saturating at 65504.
__device__ __forceinline__ uint32_t f32_to_f16_sat_bits(float f) {
  _Float16 h = (_Float16)fminf(f, 65504.0f);
  return (uint32_t)__builtin_bit_cast(unsigned short, h);
}

__device__ __forceinline__ float f16_bits_to_f32(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (unsigned short)h);
}

// fp32 (finite, >= 0) -> OCP E4M3 "FN" byte, round-to-nearest-even,
// saturating at 448.  Subnormal step 2^-9, normal exponents -6..8.
__device__ __forceinline__ uint32_t f32_to_e4m3_sat_pos(float a) {
  if (a >= 464.0f) return 0x7Eu;  // rounds beyond 448: saturate
  int e = (int)((__float_as_uint(a) >> 23) & 0xFF) - 127;
  if (e < -6) {  // subnormal range (and zero): count steps of 2^-9
    return (uint32_t)__builtin_rintf(a * 512.0f);  // 8 steps == 0x08 == 2^-6
  }
  uint32_t q = (uint32_t)__builtin_rintf(__builtin_ldexpf(a, 3 - e));  // 8..16
  if (q == 16u) { q = 8u; e += 1; }
  uint32_t code = ((uint32_t)(e + 7) << 3) | (q - 8u);
  return code > 0x7Eu ? 0x7Eu : code;
}

__device__ __forceinline__ float e4m3_to_f32(uint32_t b) {
  uint32_t m = b & 7u, e = (b >> 3) & 15u;
  float v = e ? __builtin_ldexpf(1.0f + (float)m * 0.125f, (int)e - 7) : (float)m * (1.0f / 512.0f);
  return (b & 0x80u) ? -v : v;
}

// fp32 (finite) -> E2M1 nibble, round-to-nearest-even (ties to the even code),
// saturating at 6; the sign bit follows the input, also for a zero result.
__device__ __forceinline__ uint32_t f32_to_e2m1_sat(float v) {
  float a = fabsf(v);
  uint32_t c = (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) +
               (uint32_t)(a >= 1.75f) + (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) +
               (uint32_t)(a > 5.0f);
  return c | ((__float_as_uint(v) >> 28) & 8u);
}

// ---- lane helpers ------------------------------------------------------------
__device__ __forceinline__ float shfl_xor_f(float v, int mask) {
  return __shfl_xor(v, mask, 64);
}

}  // namespace svdq
