// Device helpers of the fused attention-projection epilogue: per-head RMSNorm
// of Q and K followed by the rotary embedding, applied to the fp32 GEMM result
// before its bf16 rounding ("Nunchaku Lite", "Fused kernels"; blog "Nunchaku
// 4-bit inference in Diffusers", "Quantizing models with structural rewrites":
// one operator takes the grouped Q/K/V projection, the Q and K norms and the
// rotary embedding).
//
// In both GEMM kernels every lane holds, for each of its token columns, runs
// of four consecutive output channels, so a rotary pair (2p, 2p+1) never
// leaves the lane; only the per-token sum of squares crosses lanes (and, for
// 128-channel heads, the two waves that split a head's columns).
#pragma once

#include "common.h"
#include "launch.h"

namespace svdq {

// Sum over lanes l, l^16, l^32, l^48 (permlane swaps of whole 16-lane rows).
__device__ __forceinline__ float sum_over_rows16(float v) {
  u32 bv = __float_as_uint(v);
  auto p = __builtin_amdgcn_permlane16_swap(bv, bv, false, false);
  v = __uint_as_float(p[0]) + __uint_as_float(p[1]);
  bv = __float_as_uint(v);
  auto q = __builtin_amdgcn_permlane32_swap(bv, bv, false, false);
  return __uint_as_float(q[0]) + __uint_as_float(q[1]);
}

// Sum over lanes l and l^32.
__device__ __forceinline__ float sum_over_halves(float v) {
  const u32 bv = __float_as_uint(v);
  auto q = __builtin_amdgcn_permlane32_swap(bv, bv, false, false);
  return __uint_as_float(q[0]) + __uint_as_float(q[1]);
}

// 1 / sqrt(mean square + eps) from a head's sum of squares (head_dim is a
// power of two, so the mean is exact), with the hardware reciprocal square
// root v_rsq_f32 (about 1 ulp; the result is rounded to bf16 in the end).
__device__ __forceinline__ float inv_rms(float ss, const QkvEpi& q) {
  return __builtin_amdgcn_rsqf(ss * (1.0f / (float)q.head_dim) + q.eps);
}

// Rotary-table rows of the tokens m, m + STEP, ..., m + (NJ-1)*STEP, i.e. each
// token mod rope_rows: one division, then one conditional subtraction per
// step whenever the table is longer than the span (wave-uniform choice).
template <int NJ, int STEP>
__device__ __forceinline__ void rope_rows_of(int m, const QkvEpi& q, int (&row)[NJ]) {
  const int S = q.rope_rows;
  if (S > (NJ - 1) * STEP) {
    int r = m % S;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      row[j] = r;
      r += STEP;
      r = r >= S ? r - S : r;
    }
  } else {
#pragma unroll
    for (int j = 0; j < NJ; ++j) row[j] = (m + j * STEP) % S;
  }
}

// Four consecutive channels 4c .. 4c+3 of one head of one token: multiply by
// the token's 1/rms and the norm weights w (four bf16), then rotate the pairs
// (4c, 4c+1) and (4c+2, 4c+3) by (cos, sin) = (cs.x, cs.y) and (cs.z, cs.w).
// Without a rotary table cs is (1, 0, 1, 0), an exact identity.
__device__ __forceinline__ float4 norm_rope4(float y0, float y1, float y2, float y3, float r, uint2 w,
                                             float4 cs) {
  const float u0 = y0 * r * bf16_bits_to_f32(w.x & 0xFFFFu);
  const float u1 = y1 * r * bf16_bits_to_f32(w.x >> 16);
  const float u2 = y2 * r * bf16_bits_to_f32(w.y & 0xFFFFu);
  const float u3 = y3 * r * bf16_bits_to_f32(w.y >> 16);
  return float4{u0 * cs.x - u1 * cs.y, u0 * cs.y + u1 * cs.x, u2 * cs.z - u3 * cs.w, u2 * cs.w + u3 * cs.z};
}

// Which block of [Q | K | V] the 64-aligned column n lies in (0, 1, 2), and
// the channel of n within its head.
__device__ __forceinline__ int qkv_part(int n, const QkvEpi& q) { return n < q.hd ? 0 : n < 2 * q.hd ? 1 : 2; }
__device__ __forceinline__ int qkv_channel(int n, const QkvEpi& q) { return (n % q.hd) % q.head_dim; }

}  // namespace svdq
