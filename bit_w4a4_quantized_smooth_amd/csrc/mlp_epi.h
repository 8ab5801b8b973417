// Device helpers of the fused MLP up-projection epilogue ("Nunchaku Lite",
// "Fused kernels": the original engine fuses the GELU MLP): GELU of the fp32
// projection, rounded to bf16, then quantized for the down projection.
#pragma once

#include "common.h"

namespace svdq {

// GELU(y) = y * Phi(y) with the standard normal CDF from the rational
// approximation 7.1.26 of Abramowitz and Stegun (Handbook of Mathematical
// Functions, 1964): for x >= 0, erfc(x) = (a1 t + ... + a5 t^5) exp(-x^2) with
// t = 1 / (1 + p x), absolute error below 1.5e-7.  Phi(y) = erfc(-y/sqrt 2)/2,
// evaluated as Q/2 for y < 0 and 1 - Q/2 for y >= 0 with Q = erfc(|y|/sqrt 2),
// so there is no cancellation in the negative tail.  exp and the reciprocal
// are the hardware v_exp_f32 / v_rcp_f32 (about 1 ulp).
__device__ __forceinline__ float gelu_f32(float y) {
  const float x = fabsf(y) * 0.70710678118654752f;
  const float t = __builtin_amdgcn_rcpf(fmaf(0.3275911f, x, 1.0f));
  float p = fmaf(1.061405429f, t, -1.453152027f);
  p = fmaf(p, t, 1.421413741f);
  p = fmaf(p, t, -0.284496736f);
  p = fmaf(p, t, 0.254829592f);
  p *= t;
  const float q = p * __builtin_amdgcn_exp2f(-x * x * 1.44269504088896341f);  // erfc(x)
  const float phi = y >= 0.0f ? fmaf(-0.5f, q, 1.0f) : 0.5f * q;
  return y * phi;
}

// Max over lanes l, l^16, l^32 and l^48 (the four lanes that share a token
// column in the 16x16 matrix-core output layout).
__device__ __forceinline__ float max_over_rows16(float v) {
  u32 bv = __float_as_uint(v);
  auto p = __builtin_amdgcn_permlane16_swap(bv, bv, false, false);
  v = fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
  bv = __float_as_uint(v);
  auto q = __builtin_amdgcn_permlane32_swap(bv, bv, false, false);
  return fmaxf(__uint_as_float(q[0]), __uint_as_float(q[1]));
}

static __global__ void fill_zero_f32(float* __restrict__ p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0.0f;
}

}  // namespace svdq
