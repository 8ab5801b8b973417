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

// Eight E2M1 codes of fl32(v_i * t) in one word (code i in bits 4i .. 4i+3,
// sign in the nibble's top bit), two per v_cvt_scalef32_pk_fp4_f32 with unit
// scale.  The conversion rounds to nearest even (ties to the even code),
// saturates at 6, keeps the sign also when the magnitude rounds to zero, and
// gives the largest magnitude with the input's sign for +-inf and NaN.  That is
// the E2M1 encoding of the format definition for every fp32 input: all finite
// inputs were compared on the device against a compare-and-count rounding
// with thresholds 0.25, 0.75, 1.25, 1.75, 2.5, 3.5 and 5 (ties at the strict
// ones go down to the even code), with no difference.
__device__ __forceinline__ uint32_t e2m1_codes8(const float* v, float t) {
  uint32_t w = 0u;
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, __fmul_rn(v[0], t), __fmul_rn(v[1], t), 1.0f, 0);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, __fmul_rn(v[2], t), __fmul_rn(v[3], t), 1.0f, 1);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, __fmul_rn(v[4], t), __fmul_rn(v[5], t), 1.0f, 2);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, __fmul_rn(v[6], t), __fmul_rn(v[7], t), 1.0f, 3);
  return w;
}

// fl32(a / 7) for every non-negative finite a, without a division: q0 =
// fl32(a * fl32(1/7)), the residual a - 7 q0 exactly by an fma, then one fma
// correction.  Equal to the IEEE quotient for all 2^31 - 2^23 such a,
// subnormals included (checked exhaustively by tests/test_div7_exhaustive.py).
// a = +inf gives NaN, which the saturating fp16 conversion of the int4 scale
// maps to 65504 as it does inf.
__device__ __forceinline__ float div7_rn(float a) {
  const float r7 = 0.142857149f;  // fl32(1/7)
  const float q0 = __fmul_rn(a, r7);
  const float r = __builtin_fmaf(-q0, 7.0f, a);
  return __builtin_fmaf(r, r7, q0);
}

// Eight int4 codes q_i = clamp(rne(fl32(v_i * t)), -8, 7) as two's complement
// nibbles of one word (code i in bits 4i .. 4i+3).  Clamping to the integer
// bounds first gives the same result as clamping after rounding; then one add
// of 2^23 + 8 rounds (ties to even: the even offset keeps the parity) and
// leaves q + 8 in 0..15 as the low bits of the sum's bit pattern, with only
// exponent bits above them; those shift out for codes 2..7 and are masked
// for codes 0 and 1; one xor with 8 per nibble turns q + 8 into q's nibble.
__device__ __forceinline__ uint32_t int4_codes8(const float* v, float t) {
  uint32_t w = 0u;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float c = __builtin_amdgcn_fmed3f(__fmul_rn(v[i], t), -8.0f, 7.0f);
    const uint32_t b = __float_as_uint(__fadd_rn(c, 8388616.0f));  // 2^23 + 8 + rne(c)
    w |= (i < 2 ? (b & 0xFu) : b) << (4 * i);
  }
  return w ^ 0x88888888u;
}

// ---- lane helpers ------------------------------------------------------------
__device__ __forceinline__ float shfl_xor_f(float v, int mask) {
  return __shfl_xor(v, mask, 64);
}

}  // namespace svdq
