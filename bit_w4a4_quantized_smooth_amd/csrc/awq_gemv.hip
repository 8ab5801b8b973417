// AWQ W4A16 linear ("Nunchaku Lite", "Supported quantization types":
// awq_w4a16, int4 weight-only, group 64; blog "Nunchaku 4-bit inference in
// Diffusers", "Introducing Nunchaku Lite": memory-bound modulation
// projections):
//   y[m,n] = sum_g s[n,g] * ( sum_{k in g} x[m,k] * q[n,k]  -  z[n,g] * sum_{k in g} x[m,k] ) + bias[n]
// which equals sum_k x * (q - z) * s (the weight dequantized per group).
//
// Two kernels:
//  * M <= 2 (the decode-like case that is bound by streaming the 4-bit
//    weights): a 32-lane team owns one weight row; lane i reads the 16-byte
//    chunks i, i+32, i+64, ... so every load instruction of the team covers
//    512 contiguous bytes.  The lane's slice of x stays in registers for the
//    whole kernel as bf16 pairs.  Codes become bf16 pairs with one AND-OR
//    each: (nibble | 0x4300) is the bf16 number 128 + q, so v_dot2_f32_bf16
//    accumulates sum x*(128+q) and the 128*sum(x) term is folded into the
//    zero-point, z' = z + 128.
//  * 2 < M <= 64: matrix-core kernel, see awq_gemm_mfma_kernel.
#include "common.h"
#include "launch.h"

namespace svdq {

typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

namespace {
constexpr int AWQ_RP = 4;   // row pairs per wave
constexpr int AWQ_CPL = 4;  // 32-channel chunks per lane per pass (pass = 4096 channels)

__device__ __forceinline__ float dot2bf(u32 a, u32 b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(v2bf, a), __builtin_bit_cast(v2bf, b), c, false);
}
}  // namespace

template <int MR>
__global__ __launch_bounds__(256) void awq_gemv_kernel(
    int M, int N, int K, const uint16_t* __restrict__ x, const uint8_t* __restrict__ wc,
    const uint16_t* __restrict__ ws, const uint16_t* __restrict__ wz,
    const uint16_t* __restrict__ bias, uint16_t* __restrict__ y) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int team = lane >> 5, li = lane & 31;
  const int n_base = (blockIdx.x * 4 + wave) * (2 * AWQ_RP);
  const int G = K >> 6, nchunks = K >> 5;
  const size_t rowb = (size_t)(K >> 1);

  float acc[AWQ_RP][MR];
#pragma unroll
  for (int p = 0; p < AWQ_RP; ++p)
#pragma unroll
    for (int m = 0; m < MR; ++m) acc[p][m] = 0.0f;

  for (int cbase = 0; cbase < nchunks; cbase += 32 * AWQ_CPL) {
    // this lane's x slice as (k, k+4) bf16 pairs, plus the fp32 sum per chunk
    u32 xp[AWQ_CPL][MR][16];
    float xs[AWQ_CPL][MR];
#pragma unroll
    for (int t = 0; t < AWQ_CPL; ++t) {
      const int c = cbase + li + 32 * t;
#pragma unroll
      for (int m = 0; m < MR; ++m) {
        xs[t][m] = 0.0f;
#pragma unroll
        for (int b = 0; b < 16; ++b) xp[t][m][b] = 0u;
        if (c < nchunks && m < M) {
          const uint4* src = (const uint4*)(x + (size_t)m * K + 32 * c);
#pragma unroll
          for (int b = 0; b < 4; ++b) {  // 8 channels: words (k0,k1) (k2,k3) (k4,k5) (k6,k7)
            const uint4 w = src[b];
            xp[t][m][4 * b + 0] = __builtin_amdgcn_perm(w.z, w.x, 0x05040100u);  // (k0, k4)
            xp[t][m][4 * b + 1] = __builtin_amdgcn_perm(w.z, w.x, 0x07060302u);  // (k1, k5)
            xp[t][m][4 * b + 2] = __builtin_amdgcn_perm(w.w, w.y, 0x05040100u);  // (k2, k6)
            xp[t][m][4 * b + 3] = __builtin_amdgcn_perm(w.w, w.y, 0x07060302u);  // (k3, k7)
            const u32 ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int q = 0; q < 4; ++q)
              xs[t][m] += bf16_bits_to_f32(ww[q] & 0xFFFFu) + bf16_bits_to_f32(ww[q] >> 16);
          }
        }
      }
    }

    // stream the weight rows: all loads of the wave's rows are issued first
    uint4 wv[AWQ_RP][AWQ_CPL];
#pragma unroll
    for (int p = 0; p < AWQ_RP; ++p) {
      const int n = n_base + 2 * p + team;
#pragma unroll
      for (int t = 0; t < AWQ_CPL; ++t) {
        const int c = cbase + li + 32 * t;
        wv[p][t] = (n < N && c < nchunks) ? *(const uint4*)(wc + (size_t)n * rowb + 16 * c)
                                           : uint4{0u, 0u, 0u, 0u};
      }
    }
#pragma unroll
    for (int p = 0; p < AWQ_RP; ++p) {
      const int n = n_base + 2 * p + team;
#pragma unroll
      for (int t = 0; t < AWQ_CPL; ++t) {
        const int c = cbase + li + 32 * t;
        if (n >= N || c >= nchunks) continue;
        const int g = c >> 1;
        const float s = f16_bits_to_f32(ws[(size_t)n * G + g]);
        const float zp = f16_bits_to_f32(wz[(size_t)n * G + g]) + 128.0f;
        const u32 d4[4] = {wv[p][t].x, wv[p][t].y, wv[p][t].z, wv[p][t].w};
        float dot[MR];
#pragma unroll
        for (int m = 0; m < MR; ++m) dot[m] = 0.0f;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const u32 d = d4[b];
          const u32 q0 = (d & 0x000F000Fu) | 0x43004300u;          // (k0, k4)
          const u32 q1 = ((d >> 4) & 0x000F000Fu) | 0x43004300u;   // (k1, k5)
          const u32 q2 = ((d >> 8) & 0x000F000Fu) | 0x43004300u;   // (k2, k6)
          const u32 q3 = ((d >> 12) & 0x000F000Fu) | 0x43004300u;  // (k3, k7)
#pragma unroll
          for (int m = 0; m < MR; ++m) {
            dot[m] = dot2bf(q0, xp[t][m][4 * b + 0], dot[m]);
            dot[m] = dot2bf(q1, xp[t][m][4 * b + 1], dot[m]);
            dot[m] = dot2bf(q2, xp[t][m][4 * b + 2], dot[m]);
            dot[m] = dot2bf(q3, xp[t][m][4 * b + 3], dot[m]);
          }
        }
#pragma unroll
        for (int m = 0; m < MR; ++m) acc[p][m] = fmaf(s, fmaf(-zp, xs[t][m], dot[m]), acc[p][m]);
      }
    }
  }

  // team reduction and store
#pragma unroll
  for (int p = 0; p < AWQ_RP; ++p) {
    const int n = n_base + 2 * p + team;
#pragma unroll
    for (int m = 0; m < MR; ++m) {
      float v = acc[p][m];
#pragma unroll
      for (int o = 16; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
      if (li == 0 && n < N && m < M) {
        if (bias) v += bf16_bits_to_f32(bias[n]);
        y[(size_t)m * N + n] = (uint16_t)f32_to_bf16_bits(v);
      }
    }
  }
}

// 2 < M <= 64: D[m][n] = sum_k x[m,k] * q[n,k] per 64-channel group on the bf16
// matrix cores (both operands exact in bf16), then in fp32
//   acc[m][n] += s[n,g] * (P[m][n] - z[n,g] * xsum[m,g]).
// Workgroup: 64 weight rows x all (<= 64, zero padded) activation rows; wave w
// owns the 32x32 block (m half w&1, n half w>>1).  The matrix-core A operand
// is x (rows m) and B the weight tile (columns n), so each lane holds one
// column n: its scale and zero-point are per-lane scalars and each store of
// the 32 lanes covers 64 contiguous bytes of a Y row.
__global__ __launch_bounds__(256) void awq_gemm_mfma_kernel(
    int M, int N, int K, const uint16_t* __restrict__ x, const uint8_t* __restrict__ wc,
    const uint16_t* __restrict__ ws, const uint16_t* __restrict__ wz,
    const uint16_t* __restrict__ bias, uint16_t* __restrict__ y) {
  constexpr int ROW = 72;  // bf16 per LDS row: 64 channels + 8 padding
  __shared__ __align__(16) uint16_t sX[64 * ROW];
  __shared__ __align__(16) uint16_t sW[64 * ROW];
  __shared__ float sXS[64];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int n0 = blockIdx.x * 64;
  const int G = K >> 6;
  const size_t rowb = (size_t)(K >> 1);
  const int bm = (wave & 1) * 32, bn = (wave >> 1) * 32;
  const int lr = lane & 31, lh = lane >> 5;
  const int n = n0 + bn + lr;

  v16f acc;
#pragma unroll
  for (int v = 0; v < 16; ++v) acc[v] = 0.0f;

  // staging: x rows 64 x 64 channels (thread: row tid>>2, 16 channels);
  //          weight rows 64 x 32 bytes (thread: row tid>>2, 8 bytes = 16 codes)
  const int srow = tid >> 2, sq = tid & 3;
  for (int g = 0; g < G; ++g) {
    uint4 xa = {0u, 0u, 0u, 0u}, xb = {0u, 0u, 0u, 0u};
    if (srow < M) {
      const uint4* src = (const uint4*)(x + (size_t)srow * K + 64 * g + 16 * sq);
      xa = src[0];
      xb = src[1];
    }
    const uint2 wq = *(const uint2*)(wc + (size_t)(n0 + srow) * rowb + 32 * g + 8 * sq);
    __syncthreads();  // previous group's LDS reads are done
    *(uint4*)&sX[srow * ROW + 16 * sq] = xa;
    *(uint4*)&sX[srow * ROW + 16 * sq + 8] = xb;
    // codes -> bf16 values 0..15 (exact): 0x4300|q is 128+q, minus 128 below
    u32 wb[8];
    const u32 wq2[2] = {wq.x, wq.y};
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const u32 q0 = (wq2[h] >> (8 * e)) & 0xFu, q1 = (wq2[h] >> (8 * e + 4)) & 0xFu;
        const float f0 = (float)q0, f1 = (float)q1;
        wb[4 * h + e] = (__float_as_uint(f0) >> 16) | (__float_as_uint(f1) & 0xFFFF0000u);
      }
    *(uint4*)&sW[srow * ROW + 16 * sq] = uint4{wb[0], wb[1], wb[2], wb[3]};
    *(uint4*)&sW[srow * ROW + 16 * sq + 8] = uint4{wb[4], wb[5], wb[6], wb[7]};
    // per-row sums of x over the group (fp32), four threads per row
    float ps = 0.0f;
    const u32 xw[8] = {xa.x, xa.y, xa.z, xa.w, xb.x, xb.y, xb.z, xb.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) ps += bf16_bits_to_f32(xw[i] & 0xFFFFu) + bf16_bits_to_f32(xw[i] >> 16);
    ps += __shfl_xor(ps, 1, 64);
    ps += __shfl_xor(ps, 2, 64);
    if (sq == 0) sXS[srow] = ps;
    __syncthreads();

    v16f d;
#pragma unroll
    for (int v = 0; v < 16; ++v) d[v] = 0.0f;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const v8bf a = *(const v8bf*)&sX[(bm + lr) * ROW + 16 * kk + 8 * lh];
      const v8bf b = *(const v8bf*)&sW[(bn + lr) * ROW + 16 * kk + 8 * lh];
      d = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, d, 0, 0, 0);
    }
    const float s = f16_bits_to_f32(ws[(size_t)n * G + g]);
    const float z = f16_bits_to_f32(wz[(size_t)n * G + g]);
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int ml = bm + 8 * (v >> 2) + 4 * lh + (v & 3);
      acc[v] = fmaf(s, fmaf(-z, sXS[ml], d[v]), acc[v]);
    }
  }
  const float bv = bias ? bf16_bits_to_f32(bias[n]) : 0.0f;
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int m = bm + 8 * (v >> 2) + 4 * lh + (v & 3);
    if (m < M) y[(size_t)m * N + n] = (uint16_t)f32_to_bf16_bits(acc[v] + bv);
  }
}

hipError_t launch_awq(const AwqArgs& a, hipStream_t st) {
  const int M = (int)a.M, N = (int)a.N, K = (int)a.K;
  if (M <= 2) {
    const int rows_per_block = 4 * 2 * AWQ_RP;
    const int blocks = (N + rows_per_block - 1) / rows_per_block;
    auto kern = M == 1 ? awq_gemv_kernel<1> : awq_gemv_kernel<2>;
    hipLaunchKernelGGL(kern, dim3(blocks), dim3(256), 0, st, M, N, K, (const uint16_t*)a.x,
                       (const uint8_t*)a.w_codes, (const uint16_t*)a.w_scales,
                       (const uint16_t*)a.w_zeros, (const uint16_t*)a.bias, (uint16_t*)a.y);
  } else {
    hipLaunchKernelGGL(awq_gemm_mfma_kernel, dim3(N / 64), dim3(256), 0, st, M, N, K,
                       (const uint16_t*)a.x, (const uint8_t*)a.w_codes, (const uint16_t*)a.w_scales,
                       (const uint16_t*)a.w_zeros, (const uint16_t*)a.bias, (uint16_t*)a.y);
  }
  return hipGetLastError();
}

}  // namespace svdq
