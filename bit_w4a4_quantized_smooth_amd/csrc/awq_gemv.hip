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
//    The workgroup's scales and zero-points are staged in LDS as fp32 pairs
//    by wide coalesced loads.  All staging loads are issued before the weight
//    loads (the memory counter is in order), so block t of the codes waits
//    only for itself.  Needs K % 512 == 0 and K <= 8192.
//  * other shapes (4 < M <= 64, or K outside that range): matrix-core
//    kernel, see awq_gemm_mfma_kernel.
#include "common.h"
#include "launch.h"

namespace svdq {

typedef __bf16 v4bf __attribute__((ext_vector_type(4)));

namespace {
constexpr uint32_t kBufDword3 = 0x00020000u;  // raw buffer, 32-bit data format
constexpr int kOut = 0x7FFFFFF0;              // offset past num_records: the load returns 0
constexpr int AWQ_WAVES = 8;                  // small-M kernel: waves per workgroup
constexpr int AWQ_RQ = 1;                     // row quads per wave
constexpr int AWQ_ROWS = 4 * AWQ_RQ * AWQ_WAVES;  // weight rows per workgroup (power of 2)
constexpr int AWQ_LOG_ROWS = AWQ_ROWS == 32 ? 5 : AWQ_ROWS == 64 ? 6 : 7;
constexpr int AWQ_NT = 64 * AWQ_WAVES;
constexpr int AWQ_PT = 6;                     // 512-channel blocks whose codes are loaded together
constexpr int AWQ_TBMAX = 16;                 // K <= 8192
constexpr int AWQ_SS = (AWQ_ROWS * AWQ_TBMAX + AWQ_NT - 1) / AWQ_NT;  // scale items per thread

__device__ __forceinline__ v4bf as_v4bf(u32 lo, u32 hi) {
  return __builtin_bit_cast(v4bf, uint2{lo, hi});
}

// A constant the compiler cannot fold into an instruction: the three-operand
// AND-OR takes no literal on this target, so the masks live in registers.
__device__ __forceinline__ u32 in_vgpr(u32 v) {
  u32 r;
  asm("v_mov_b32 %0, %1" : "=v"(r) : "i"(v));
  return r;
}

// LDS of the small-M kernel, in bytes: x as pairs [TB][4 words][16][MR]
// (16 B each), the per-chunk sums of x [TB*16][MR] (fp32), the workgroup's
// (scale, zero-point + 128) pairs [AWQ_ROWS][G] (fp32), and a spare slot
// that takes the stores of staging items past the end.
struct AwqLds {
  int xsl, sz, trash, total, nx, ns;  // nx: 16-byte x items; ns: 8-group scale items
};
__host__ __device__ inline AwqLds awq_lds(int K, int MR) {
  const int TB = K / 512, G = K / 64;
  AwqLds L;
  L.xsl = TB * 64 * MR * 16;
  L.sz = L.xsl + TB * 16 * MR * 4;
  L.trash = L.sz + AWQ_ROWS * G * 8;
  L.total = L.trash + 64;
  L.nx = MR * TB * 64;
  L.ns = AWQ_ROWS * TB;
  return L;
}
}  // namespace

// Requires K % 512 == 0 (every 16-lane load of a row is whole), K <= 8192,
// N % AWQ_ROWS == 0 and M <= MR.
template <int MR, int SX>
__global__ __launch_bounds__(AWQ_NT) void awq_gemv_kernel(
    int M, int N, int K, const uint16_t* __restrict__ x, const uint8_t* __restrict__ wc,
    const uint16_t* __restrict__ ws, const uint16_t* __restrict__ wz,
    const uint16_t* __restrict__ bias, uint16_t* __restrict__ y) {
  extern __shared__ __align__(16) uint4 lds4[];
  const int TB = K >> 9, G = K >> 6, rowb = K >> 1;
  const AwqLds L = awq_lds(K, MR);
  uint8_t* lds = (uint8_t*)lds4;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int b = lane >> 2, c = lane & 3;
  const int n0 = blockIdx.x * AWQ_ROWS;
  const int arow = c % MR;  // A rows past MR only feed D rows that are never read
  const __amdgpu_buffer_rsrc_t xres = __builtin_amdgcn_make_buffer_rsrc((void*)x, (short)0, M * K * 2, kBufDword3);
  const __amdgpu_buffer_rsrc_t wres = __builtin_amdgcn_make_buffer_rsrc((void*)wc, (short)0, N * rowb, kBufDword3);
  const __amdgpu_buffer_rsrc_t sres = __builtin_amdgcn_make_buffer_rsrc((void*)ws, (short)0, N * G * 2, kBufDword3);
  const __amdgpu_buffer_rsrc_t zres = __builtin_amdgcn_make_buffer_rsrc((void*)wz, (short)0, N * G * 2, kBufDword3);

  // Staging loads, issued before the weight loads so that waiting for them
  // (the counter is in order) does not wait for the weights.  x item
  // it = ((m * TB + t) * 16 + chunk-in-block) * 4 + word; scale item
  // q = 8-group block * AWQ_ROWS + row.  Items past the end read zeros.
  uint4 xw[SX];
#pragma unroll
  for (int j = 0; j < SX; ++j) {
    const int it = tid + j * AWQ_NT;
    int m = 0, tt = it >> 6;
#pragma unroll
    for (int e = 1; e < MR; ++e)
      if (tt >= TB) { tt -= TB; ++m; }
    const int ch = (tt << 4) + ((it >> 2) & 15);
    const bool ok = it < L.nx && m < M;
    xw[j] = __builtin_bit_cast(
        uint4, __builtin_amdgcn_raw_buffer_load_b128(xres, ok ? (m * K + 32 * ch + 8 * (it & 3)) * 2 : kOut, 0, 0));
  }
  uint4 sr[AWQ_SS], zr[AWQ_SS];
#pragma unroll
  for (int j = 0; j < AWQ_SS; ++j) {
    const int q = tid + j * AWQ_NT;
    const int off = q < L.ns ? ((n0 + (q & (AWQ_ROWS - 1))) * G + 8 * (q >> AWQ_LOG_ROWS)) * 2 : kOut;
    sr[j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(sres, off, 0, 0));
    zr[j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(zres, off, 0, 0));
  }

  // codes of this lane's chunks in blocks t0 .. t0+AWQ_PT-1 for its rows,
  // block-major so that block u waits only for its own loads
  uint4 cv[AWQ_PT][AWQ_RQ];
  auto load_pass = [&](int t0) {
#pragma unroll
    for (int u = 0; u < AWQ_PT; ++u)
#pragma unroll
      for (int q = 0; q < AWQ_RQ; ++q) {
        const int n = n0 + wave * 4 * AWQ_RQ + 4 * q + c;
        cv[u][q] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                                 wres, t0 + u < TB ? n * rowb + 16 * (16 * (t0 + u) + b) : kOut, 0, 0));
      }
  };
  load_pass(0);

  // x as (k, k+4) bf16 pairs in the order the codes are expanded below, and
  // its fp32 sum per 32-channel chunk.  Stores are unconditional (items past
  // the end go to the spare slot).
#pragma unroll
  for (int j = 0; j < SX; ++j) {
    const int it = tid + j * AWQ_NT;
    int m = 0, tt = it >> 6;
#pragma unroll
    for (int e = 1; e < MR; ++e)
      if (tt >= TB) { tt -= TB; ++m; }
    const int i = it & 3, bb = (it >> 2) & 15;
    const bool live = it < L.nx;
    const uint4 w = xw[j];
    const uint4 pr = {__builtin_amdgcn_perm(w.z, w.x, 0x05040100u),   // (k0, k4)
                      __builtin_amdgcn_perm(w.z, w.x, 0x07060302u),   // (k1, k5)
                      __builtin_amdgcn_perm(w.w, w.y, 0x05040100u),   // (k2, k6)
                      __builtin_amdgcn_perm(w.w, w.y, 0x07060302u)};  // (k3, k7)
    *(uint4*)(lds + (live ? (((tt * 4 + i) * 16 + bb) * MR + m) * 16 : L.trash)) = pr;
    float sm = bf16_bits_to_f32(w.x & 0xFFFFu) + bf16_bits_to_f32(w.x >> 16);
    sm += bf16_bits_to_f32(w.y & 0xFFFFu) + bf16_bits_to_f32(w.y >> 16);
    sm += bf16_bits_to_f32(w.z & 0xFFFFu) + bf16_bits_to_f32(w.z >> 16);
    sm += bf16_bits_to_f32(w.w & 0xFFFFu) + bf16_bits_to_f32(w.w >> 16);
    // the four words of a chunk are adjacent lanes: sum them with quad DPP moves
    sm += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, sm), 0xB1, 0xF, 0xF, false));
    sm += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, sm), 0x4E, 0xF, 0xF, false));
    *(float*)(lds + (live && i == 0 ? L.xsl + 4 * (((tt << 4) + bb) * MR + m) : L.trash + 16)) = sm;
  }
  // (scale, zero-point + 128) as fp32 pairs
#pragma unroll
  for (int j = 0; j < AWQ_SS; ++j) {
    const int q = tid + j * AWQ_NT;
    const bool live = q < L.ns;
    const u32 sw4[4] = {sr[j].x, sr[j].y, sr[j].z, sr[j].w}, zw4[4] = {zr[j].x, zr[j].y, zr[j].z, zr[j].w};
    float4 o[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      o[e] = float4{f16_bits_to_f32(sw4[e] & 0xFFFFu), f16_bits_to_f32(zw4[e] & 0xFFFFu) + 128.0f,
                    f16_bits_to_f32(sw4[e] >> 16), f16_bits_to_f32(zw4[e] >> 16) + 128.0f};
    float4* dst = (float4*)(lds + (live ? L.sz + ((q & (AWQ_ROWS - 1)) * G + 8 * (q >> AWQ_LOG_ROWS)) * 8 : L.trash));
    const int step = live ? 1 : 0;  // the spare slot takes all four
#pragma unroll
    for (int e = 0; e < 4; ++e) dst[e * step] = o[e];
  }
  __syncthreads();

  const uint4* xl = lds4;
  const float* xsl = (const float*)(lds + L.xsl);
  const float2* szl = (const float2*)(lds + L.sz);
  const u32 kMask = in_vgpr(0x000F000Fu), kBf128 = in_vgpr(0x43004300u);

  float acc[AWQ_RQ][MR];
#pragma unroll
  for (int q = 0; q < AWQ_RQ; ++q)
#pragma unroll
    for (int v = 0; v < MR; ++v) acc[q][v] = 0.0f;

  for (int t0 = 0;;) {
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
#pragma unroll
      for (int q = 0; q < AWQ_RQ; ++q) {
        const int r = wave * 4 * AWQ_RQ + 4 * q + c;
        const float2 sz = szl[r * G + 8 * t + (b >> 1)];
        const u32 d4[4] = {cv[u][q].x, cv[u][q].y, cv[u][q].z, cv[u][q].w};
        v4f d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const u32 w = d4[i];
          const u32 q0 = (w & kMask) | kBf128;          // (k0, k4)
          const u32 q1 = ((w >> 4) & kMask) | kBf128;   // (k1, k5)
          const u32 q2 = ((w >> 8) & kMask) | kBf128;   // (k2, k6)
          const u32 q3 = ((w >> 12) & kMask) | kBf128;  // (k3, k7)
          d = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(as_v4bf(a[i].x, a[i].y), as_v4bf(q0, q1), d, 0, 0, 0);
          d = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(as_v4bf(a[i].z, a[i].w), as_v4bf(q2, q3), d, 0, 0, 0);
        }
#pragma unroll
        for (int v = 0; v < MR; ++v) acc[q][v] = fmaf(sz.x, fmaf(-sz.y, xs[v], d[v]), acc[q][v]);
      }
    }
    t0 += AWQ_PT;
    if (t0 >= TB) break;
    load_pass(t0);
  }

  // sum over the 16 blocks (lanes c, c+4, ..., c+60), then lanes 0..3 store
#pragma unroll
  for (int q = 0; q < AWQ_RQ; ++q)
#pragma unroll
    for (int v = 0; v < MR; ++v) {
      float r = acc[q][v];
      r += __shfl_xor(r, 4, 64);
      r += __shfl_xor(r, 8, 64);
      r += __shfl_xor(r, 16, 64);
      r += __shfl_xor(r, 32, 64);
      acc[q][v] = r;
    }
  if (b == 0) {
#pragma unroll
    for (int q = 0; q < AWQ_RQ; ++q) {
      const int n = n0 + wave * 4 * AWQ_RQ + 4 * q + c;
      const float bv = bias ? bf16_bits_to_f32(bias[n]) : 0.0f;
#pragma unroll
      for (int v = 0; v < MR; ++v)
        if (v < M) y[(size_t)v * N + n] = (uint16_t)f32_to_bf16_bits(acc[q][v] + bv);
    }
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
  const AwqLds L = awq_lds(K, MR);
  const int si = (L.nx + AWQ_NT - 1) / AWQ_NT;  // x staging items per thread
  if (M <= 4 && K % 512 == 0 && K / 512 <= AWQ_TBMAX && L.total <= 64 * 1024 && si <= 8 && N % AWQ_ROWS == 0) {
    using Kern = void (*)(int, int, int, const uint16_t*, const uint8_t*, const uint16_t*, const uint16_t*,
                          const uint16_t*, uint16_t*);
    static const Kern table[3][4] = {
        {awq_gemv_kernel<1, 1>, awq_gemv_kernel<1, 2>, awq_gemv_kernel<1, 4>, awq_gemv_kernel<1, 8>},
        {awq_gemv_kernel<2, 1>, awq_gemv_kernel<2, 2>, awq_gemv_kernel<2, 4>, awq_gemv_kernel<2, 8>},
        {awq_gemv_kernel<4, 1>, awq_gemv_kernel<4, 2>, awq_gemv_kernel<4, 4>, awq_gemv_kernel<4, 8>}};
    const int sidx = si <= 1 ? 0 : si <= 2 ? 1 : si <= 4 ? 2 : 3;
    hipLaunchKernelGGL(table[MR == 1 ? 0 : MR == 2 ? 1 : 2][sidx], dim3(N / AWQ_ROWS), dim3(AWQ_NT), L.total, st,
                       M, N, K, (const uint16_t*)a.x, (const uint8_t*)a.w_codes, (const uint16_t*)a.w_scales,
                       (const uint16_t*)a.w_zeros, (const uint16_t*)a.bias, (uint16_t*)a.y);
  } else {
    hipLaunchKernelGGL(awq_gemm_mfma_kernel, dim3(N / 64), dim3(256), 0, st, M, N, K,
                       (const uint16_t*)a.x, (const uint8_t*)a.w_codes, (const uint16_t*)a.w_scales,
                       (const uint16_t*)a.w_zeros, (const uint16_t*)a.bias, (uint16_t*)a.y);
  }
  return hipGetLastError();
}

}  // namespace svdq
