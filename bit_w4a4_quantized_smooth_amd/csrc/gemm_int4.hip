// W4A4 int4 GEMM of the SVDQuant linear with per-group dequantization and the
// low-rank up-projection and bias fused into the epilogue (blog "Nunchaku
// 4-bit inference in Diffusers", "Background: SVDQuant and Nunchaku"; int4 /
// group 64 from "Nunchaku Lite", "Supported quantization types").
//
//   y[m,n] = sum_g sa[m,g] * sw[n,g] * P[m,n,g] + sum_j XL1[m,j] L2[j,n] + bias[n]
//   P[m,n,g] = sum_{k in g} qa[m,k] * qw[n,k]                    (exact int32)
//
// Tiling: a 256-thread workgroup computes a 128(n) x 128(m) tile of Y^T; each
// wave64 owns 64x64 = 2x2 blocks of v_mfma_i32_32x32x32_i8.  The matrix-core
// A operand is the weight tile (rows n) and B the activation tile (columns m),
// so every lane ends up holding one output row m and runs of four adjacent n:
// the bf16 epilogue writes 8-byte pieces of Y rows.
//
// Per 64-channel group the workgroup stages both 128x64 code tiles through
// LDS (double buffered).  Nibbles are expanded while staging: the two's
// complement nibble placed in the high half of a byte is the int8 value 16*q,
// obtained with a mask (odd channels) or a shift and mask (even channels), no
// sign extension.  Both operands get the same channel permutation, so the
// group dot product is unchanged and the matrix core returns 256*P exactly.
#include "common.h"
#include "launch.h"

namespace svdq {

namespace {
constexpr int BM = 128, BN = 128;
constexpr int LDS_ROW = 80;  // 64 int8 channels + 16 bytes of padding per row

__device__ __forceinline__ uint4 nib_lo16(uint4 v) {  // 16*q of even channels
  return uint4{(v.x << 4) & 0xF0F0F0F0u, (v.y << 4) & 0xF0F0F0F0u, (v.z << 4) & 0xF0F0F0F0u,
               (v.w << 4) & 0xF0F0F0F0u};
}
__device__ __forceinline__ uint4 nib_hi16(uint4 v) {  // 16*q of odd channels
  return uint4{v.x & 0xF0F0F0F0u, v.y & 0xF0F0F0F0u, v.z & 0xF0F0F0F0u, v.w & 0xF0F0F0F0u};
}
}  // namespace

template <int MODE>  // 0: Y = bf16 linear output; 1: int32 partial products
__global__ __launch_bounds__(256) void gemm_int4_kernel(
    int M, int N, int K, int rank, const uint8_t* __restrict__ ac, const uint16_t* __restrict__ as,
    const uint8_t* __restrict__ wc, const uint16_t* __restrict__ ws, const float* __restrict__ xl1,
    const uint16_t* __restrict__ l2t, const uint16_t* __restrict__ bias, uint16_t* __restrict__ y,
    int32_t* __restrict__ psums) {
  __shared__ __align__(16) uint8_t sW[2][BN * LDS_ROW];
  __shared__ __align__(16) uint8_t sX[2][BM * LDS_ROW];
  __shared__ __align__(16) float sSW[2][BN];
  __shared__ __align__(16) float sSA[2][BM];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int m_tiles = (M + BM - 1) / BM;
  const int mt = blockIdx.x % m_tiles, nt = blockIdx.x / m_tiles;
  const int m0 = mt * BM, n0 = nt * BN;
  const int wn = (wave >> 1) * 64, wm = (wave & 1) * 64;
  const int G = K >> 6;
  const size_t rowb = (size_t)(K >> 1);

  // staging: thread -> (row, 16-byte half of the 32-byte group slice)
  const int srow = tid >> 1, shalf = tid & 1;
  const uint8_t* wsrc = wc + (size_t)(n0 + srow) * rowb + shalf * 16;
  const bool xvalid = (m0 + srow) < M;
  const uint8_t* xsrc = ac + (size_t)(xvalid ? m0 + srow : 0) * rowb + shalf * 16;
  const int srow_s = tid & 127;
  const bool s_is_w = tid < 128;
  const bool s_valid = s_is_w || (m0 + srow_s) < M;
  const uint16_t* ssrc = MODE == 1 ? nullptr
                         : s_is_w ? ws + (size_t)(n0 + srow_s) * G
                                  : as + (size_t)(s_valid ? m0 + srow_s : 0) * G;

  v16f acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  uint4 wv, xv;
  float sv = 0.0f;
  auto gload = [&](int g) {
    wv = *(const uint4*)(wsrc + g * 32);
    xv = xvalid ? *(const uint4*)(xsrc + g * 32) : uint4{0u, 0u, 0u, 0u};
    if constexpr (MODE == 0) sv = s_valid ? f16_bits_to_f32(ssrc[g]) : 0.0f;
  };
  auto sstore = [&](int buf) {
    uint8_t* dw = &sW[buf][srow * LDS_ROW + shalf * 32];
    *(uint4*)dw = nib_lo16(wv);
    *(uint4*)(dw + 16) = nib_hi16(wv);
    uint8_t* dx = &sX[buf][srow * LDS_ROW + shalf * 32];
    *(uint4*)dx = nib_lo16(xv);
    *(uint4*)(dx + 16) = nib_hi16(xv);
    if constexpr (MODE == 0) {
      if (s_is_w) sSW[buf][srow_s] = sv;
      else sSA[buf][srow_s] = sv * (1.0f / 256.0f);  // undo the 16*16 code scaling
    }
  };

  const int lr = lane & 31, lh = lane >> 5;
  gload(0);
  sstore(0);
  __syncthreads();

  for (int g = 0; g < G; ++g) {
    const int buf = g & 1;
    if (g + 1 < G) gload(g + 1);

    v4i a[2][2], b[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        a[i][h] = *(const v4i*)&sW[buf][(wn + 32 * i + lr) * LDS_ROW + 32 * h + 16 * lh];
        b[i][h] = *(const v4i*)&sX[buf][(wm + 32 * i + lr) * LDS_ROW + 32 * h + 16 * lh];
      }

#pragma unroll
    for (int i = 0; i < 2; ++i) {
      float swv[16];
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *(float4*)&swv[4 * q] = *(const float4*)&sSW[buf][wn + 32 * i + 8 * q + 4 * lh];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        v16i d = {0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
        d = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[i][0], b[j][0], d, 0, 0, 0);
        d = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[i][1], b[j][1], d, 0, 0, 0);
        if constexpr (MODE == 1) {
          const int m = m0 + wm + 32 * j + lr;
          if (m < M) {
#pragma unroll
            for (int v = 0; v < 16; ++v) {
              const int n = n0 + wn + 32 * i + 8 * (v >> 2) + 4 * lh + (v & 3);
              psums[((size_t)m * N + n) * G + g] = d[v] >> 8;
            }
          }
        } else {
          const float sa = sSA[buf][wm + 32 * j + lr];
#pragma unroll
          for (int v = 0; v < 16; ++v) acc[i][j][v] = fmaf((float)d[v], swv[v] * sa, acc[i][j][v]);
        }
      }
    }

    if (g + 1 < G) sstore(buf ^ 1);
    __syncthreads();
  }

  if constexpr (MODE == 0) {
    // low-rank up-projection on the bf16 matrix cores: acc += L2^T[n, :] . XL1[m, :]
    for (int jb = 0; jb < rank; jb += 16) {
      v8bf al[2], bl[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        al[i] = *(const v8bf*)(l2t + (size_t)(n0 + wn + 32 * i + lr) * rank + jb + 8 * lh);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int m = m0 + wm + 32 * j + lr;
        uint4 pk = {0u, 0u, 0u, 0u};
        if (m < M) {
          const float4* src = (const float4*)(xl1 + (size_t)m * rank + jb + 8 * lh);
          const float4 f0 = src[0], f1 = src[1];
          pk.x = f32_to_bf16_bits(f0.x) | (f32_to_bf16_bits(f0.y) << 16);
          pk.y = f32_to_bf16_bits(f0.z) | (f32_to_bf16_bits(f0.w) << 16);
          pk.z = f32_to_bf16_bits(f1.x) | (f32_to_bf16_bits(f1.y) << 16);
          pk.w = f32_to_bf16_bits(f1.z) | (f32_to_bf16_bits(f1.w) << 16);
        }
        bl[j] = __builtin_bit_cast(v8bf, pk);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al[i], bl[j], acc[i][j], 0, 0, 0);
    }
    // bias, bf16 rounding, 8-byte stores of four adjacent n
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int m = m0 + wm + 32 * j + lr;
        if (m >= M) continue;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int n = n0 + wn + 32 * i + 8 * q + 4 * lh;
          float bv[4] = {0.f, 0.f, 0.f, 0.f};
          if (bias) {
            const uint2 bb = *(const uint2*)(bias + n);
            bv[0] = bf16_bits_to_f32(bb.x & 0xFFFFu);
            bv[1] = bf16_bits_to_f32(bb.x >> 16);
            bv[2] = bf16_bits_to_f32(bb.y & 0xFFFFu);
            bv[3] = bf16_bits_to_f32(bb.y >> 16);
          }
          uint2 o;
          o.x = f32_to_bf16_bits(acc[i][j][4 * q] + bv[0]) | (f32_to_bf16_bits(acc[i][j][4 * q + 1] + bv[1]) << 16);
          o.y = f32_to_bf16_bits(acc[i][j][4 * q + 2] + bv[2]) | (f32_to_bf16_bits(acc[i][j][4 * q + 3] + bv[3]) << 16);
          *(uint2*)(y + (size_t)m * N + n) = o;
        }
      }
  }
}

hipError_t launch_gemm_int4(const GemmArgs& a, hipStream_t st) {
  const int m_tiles = (int)((a.M + BM - 1) / BM);
  const int blocks = m_tiles * (int)(a.N / BN);
  if (a.psums) {
    hipLaunchKernelGGL(gemm_int4_kernel<1>, dim3(blocks), dim3(256), 0, st, (int)a.M, (int)a.N,
                       (int)a.K, 0, (const uint8_t*)a.act_codes, nullptr, (const uint8_t*)a.w_codes,
                       nullptr, nullptr, nullptr, nullptr, nullptr, (int32_t*)a.psums);
  } else {
    hipLaunchKernelGGL(gemm_int4_kernel<0>, dim3(blocks), dim3(256), 0, st, (int)a.M, (int)a.N,
                       (int)a.K, a.rank, (const uint8_t*)a.act_codes, (const uint16_t*)a.act_scales,
                       (const uint8_t*)a.w_codes, (const uint16_t*)a.w_scales, a.xl1,
                       (const uint16_t*)a.l2t, (const uint16_t*)a.bias, (uint16_t*)a.y, nullptr);
  }
  return hipGetLastError();
}

}  // namespace svdq
