// AWQ W4A16 linear ("Nunchaku Lite", "Supported quantization types":
// awq_w4a16, int4 weight-only, group 64; blog "Nunchaku 4-bit inference in
// Diffusers", "Introducing Nunchaku Lite": memory-bound modulation
// projections):
//   y[m,n] = sum_g s[n,g] * ( sum_{k in g} x[m,k] * q[n,k]  -  z[n,g] * sum_{k in g} x[m,k] ) + bias[n]
// which equals sum_k x * (q - z) * s (the weight dequantized per group).
//
// Two kernels:
//  * M <= 4 (the decode-like case, bound by streaming the 4-bit weights):
//    v_mfma_f32_4x4x4_16b_bf16, whose sixteen independent 4x4 blocks fit a
//    handful of activation rows.  Lane l = 4b + c of a wave owns weight row
//    n0 + c and the 16-byte chunks b, b+16, b+32, ... of it (the 16 lanes of
//    a row read 256 contiguous bytes per load), and holds activation row c
//    of block b as the A operand.  Each 16-byte chunk (32 codes, half a
//    group) is eight MFMAs whose block result is that chunk's partial dot
//    product for all activation rows, scaled right away by its group's scale
//    and zero-point.  Codes become bf16 pairs with one AND-OR each:
//    (nibble | 0x4300) is the bf16 number 128 + q, taking the channels of a
//    32-bit word in the order (k0,k4) (k1,k5) (k2,k6) (k3,k7); x is staged
//    once per workgroup in LDS in that same pair order, with its per-chunk
//    sums, and the 128*sum(x) term is folded into the zero-point, z' = z + 128.
//  * 4 < M <= 64: matrix-core kernel, see awq_gemm_mfma_kernel.
#include "common.h"
#include "launch.h"

namespace svdq {

typedef __bf16 v4bf __attribute__((ext_vector_type(4)));

namespace {
constexpr uint32_t kBufDword3 = 0x00020000u;  // raw buffer, 32-bit data format
constexpr int kOut = 0x7FFFFFF0;              // offset past num_records: the load returns 0
constexpr int AWQ_WAVES = 8;                  // small-M kernel: waves per workgroup
constexpr int AWQ_ROWS = 4 * AWQ_WAVES;       // weight rows per workgroup
constexpr int AWQ_PT = 6;                     // 512-channel blocks whose loads are issued together

__device__ __forceinline__ v4bf as_v4bf(u32 lo, u32 hi) {
  return __builtin_bit_cast(v4bf, uint2{lo, hi});
}

// LDS bytes of the small-M kernel: pair-permuted x and per-chunk sums.
__host__ __device__ constexpr int awq_small_lds(int K, int MR) {
  return ((K / 32 + 15) / 16) * MR * (64 * 16 + 16 * 4);
}
}  // namespace

template <int MR>
__global__ __launch_bounds__(64 * AWQ_WAVES) void awq_gemv_kernel(
    int M, int N, int K, const uint16_t* __restrict__ x, const uint8_t* __restrict__ wc,
    const uint16_t* __restrict__ ws, const uint16_t* __restrict__ wz,
    const uint16_t* __restrict__ bias, uint16_t* __restrict__ y) {
  extern __shared__ __align__(16) uint4 lds4[];
  const int nchunks = K >> 5, TB = (nchunks + 15) >> 4, G = K >> 6, rowb = K >> 1;
  uint4* xl = lds4;                        // [TB][4 words][16 blocks][MR] x pairs
  float* xsl = (float*)(lds4 + TB * 64 * MR);  // [TB*16 chunks][MR] sums of x per chunk
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int b = lane >> 2, c = lane & 3;
  const int n = blockIdx.x * AWQ_ROWS + wave * 4 + c;  // N is a multiple of AWQ_ROWS
  const int arow = c % MR;  // A rows past MR only feed D rows that are never read
  const __amdgpu_buffer_rsrc_t xres = __builtin_amdgcn_make_buffer_rsrc((void*)x, (short)0, M * K * 2, kBufDword3);
  const __amdgpu_buffer_rsrc_t wres = __builtin_amdgcn_make_buffer_rsrc((void*)wc, (short)0, N * rowb, kBufDword3);
  const __amdgpu_buffer_rsrc_t sres = __builtin_amdgcn_make_buffer_rsrc((void*)ws, (short)0, N * G * 2, kBufDword3);
  const __amdgpu_buffer_rsrc_t zres = __builtin_amdgcn_make_buffer_rsrc((void*)wz, (short)0, N * G * 2, kBufDword3);

  float acc[MR];
#pragma unroll
  for (int v = 0; v < MR; ++v) acc[v] = 0.0f;

  for (int t0 = 0; t0 < TB; t0 += AWQ_PT) {
    // codes, scales and zero-points of this lane's chunks in the next AWQ_PT
    // blocks, all in flight at once; chunks past K read as zeros
    uint4 cv[AWQ_PT];
    u32 sv[AWQ_PT], zv[AWQ_PT];
#pragma unroll
    for (int u = 0; u < AWQ_PT; ++u) {
      const int ch = 16 * (t0 + u) + b;
      const bool ok = ch < nchunks;
      cv[u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(wres, ok ? n * rowb + 16 * ch : kOut, 0, 0));
      const int go = ok ? (n * G + (ch >> 1)) * 2 : kOut;
      sv[u] = __builtin_amdgcn_raw_buffer_load_b16(sres, go, 0, 0);
      zv[u] = __builtin_amdgcn_raw_buffer_load_b16(zres, go, 0, 0);
    }

    if (t0 == 0) {
      // stage x while the first codes are in flight: item = (row m, chunk, word i)
      const int items = MR * TB * 64;
      for (int it = tid; it < items; it += 64 * AWQ_WAVES) {
        const int i = it & 3, ch = (it >> 2) % (TB * 16), m = it / (TB * 64);
        const bool ok = m < M && ch < nchunks;
        const uint4 w = __builtin_bit_cast(
            uint4, __builtin_amdgcn_raw_buffer_load_b128(xres, ok ? (m * K + 32 * ch + 8 * i) * 2 : kOut, 0, 0));
        uint4 pr;
        pr.x = __builtin_amdgcn_perm(w.z, w.x, 0x05040100u);  // (k0, k4)
        pr.y = __builtin_amdgcn_perm(w.z, w.x, 0x07060302u);  // (k1, k5)
        pr.z = __builtin_amdgcn_perm(w.w, w.y, 0x05040100u);  // (k2, k6)
        pr.w = __builtin_amdgcn_perm(w.w, w.y, 0x07060302u);  // (k3, k7)
        xl[(((ch >> 4) * 4 + i) * 16 + (ch & 15)) * MR + m] = pr;
        const u32 ww[4] = {w.x, w.y, w.z, w.w};
        float sm = 0.0f;
#pragma unroll
        for (int q = 0; q < 4; ++q) sm += bf16_bits_to_f32(ww[q] & 0xFFFFu) + bf16_bits_to_f32(ww[q] >> 16);
        sm += __shfl_xor(sm, 1, 64);  // the four words of a chunk are adjacent items
        sm += __shfl_xor(sm, 2, 64);
        if (i == 0) xsl[ch * MR + m] = sm;
      }
      __syncthreads();
    }

#pragma unroll
    for (int u = 0; u < AWQ_PT; ++u) {
      const int t = t0 + u;
      if (t >= TB) break;  // wave-uniform
      const uint4* ap = xl + (t * 64 + b) * MR + arow;
      uint4 a[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = ap[i * 16 * MR];
      float xs[MR];
#pragma unroll
      for (int v = 0; v < MR; ++v) xs[v] = xsl[(16 * t + b) * MR + v];
      const u32 d4[4] = {cv[u].x, cv[u].y, cv[u].z, cv[u].w};
      v4f d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const u32 w = d4[i];
        const u32 q0 = (w & 0x000F000Fu) | 0x43004300u;          // (k0, k4)
        const u32 q1 = ((w >> 4) & 0x000F000Fu) | 0x43004300u;   // (k1, k5)
        const u32 q2 = ((w >> 8) & 0x000F000Fu) | 0x43004300u;   // (k2, k6)
        const u32 q3 = ((w >> 12) & 0x000F000Fu) | 0x43004300u;  // (k3, k7)
        d = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(as_v4bf(a[i].x, a[i].y), as_v4bf(q0, q1), d, 0, 0, 0);
        d = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(as_v4bf(a[i].z, a[i].w), as_v4bf(q2, q3), d, 0, 0, 0);
      }
      // a chunk past K read a zero scale (and x is zero there): it adds 0
      const float s = f16_bits_to_f32(sv[u]);
      const float zp = f16_bits_to_f32(zv[u]) + 128.0f;
#pragma unroll
      for (int v = 0; v < MR; ++v) acc[v] = fmaf(s, fmaf(-zp, xs[v], d[v]), acc[v]);
    }
  }

  // sum over the 16 blocks (lanes c, c+4, ..., c+60), then lanes 0..3 store
#pragma unroll
  for (int v = 0; v < MR; ++v) {
    float r = acc[v];
    r += __shfl_xor(r, 4, 64);
    r += __shfl_xor(r, 8, 64);
    r += __shfl_xor(r, 16, 64);
    r += __shfl_xor(r, 32, 64);
    acc[v] = r;
  }
  if (b == 0) {
    const float bv = bias ? bf16_bits_to_f32(bias[n]) : 0.0f;
#pragma unroll
    for (int v = 0; v < MR; ++v)
      if (v < M) y[(size_t)v * N + n] = (uint16_t)f32_to_bf16_bits(acc[v] + bv);
  }
}

// 4 < M <= 64 (or a K too long for the small kernel's LDS): D[m][n] = sum_k x[m,k] * q[n,k] per 64-channel group on the bf16
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
  const int MR = M <= 1 ? 1 : M <= 2 ? 2 : 4;
  const int lds = awq_small_lds(K, MR);
  if (M <= 4 && lds <= 64 * 1024) {
    auto kern = MR == 1 ? awq_gemv_kernel<1> : MR == 2 ? awq_gemv_kernel<2> : awq_gemv_kernel<4>;
    hipLaunchKernelGGL(kern, dim3(N / AWQ_ROWS), dim3(64 * AWQ_WAVES), lds, st, M, N, K, (const uint16_t*)a.x,
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
