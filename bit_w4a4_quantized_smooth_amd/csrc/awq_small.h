// The small-M AWQ W4A16 kernel (M <= 4, K % 512 == 0) as an inlinable body,
// shared by its own launch (awq_gemv.hip) and the fused quantizer + GEMV
// launch (quant_act.hip), with the helpers the AWQ kernels share.  The
// formulation and layouts are described in awq_gemv.hip.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"

namespace svdq {

typedef __bf16 v4bf __attribute__((ext_vector_type(4)));

namespace {
constexpr uint32_t kBufDword3 = 0x00020000u;  // raw buffer, 32-bit data format
constexpr int kOut = 0x7FFFFFF0;              // offset past num_records: the load returns 0
// Small-M kernel: W waves per workgroup (W = 4, 6 or 8, chosen per shape so
// that the workgroups spread evenly over the 256 CUs), each owning 4 weight
// rows, so a workgroup covers 4W rows.
constexpr int AWQ_PT = 6;                     // 512-channel blocks whose codes are loaded together
constexpr int AWQ_TBMAX = 16;                 // K <= 8192

typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
constexpr u32 kOnes2 = 0x3F803F80u;  // the bf16 pair (1, 1)
__device__ __forceinline__ float dot2bf(u32 a, u32 b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(v2bf, a), __builtin_bit_cast(v2bf, b), c, false);
}

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
// (scale, zero-point + 128) pairs [rows][G] (fp32), and a spare slot that
// takes the stores of staging items past the end.
struct AwqLds {
  int xsl, sz, trash, total, nx, ns;  // nx: 16-byte x items; ns: 8-group scale items
};
__host__ __device__ inline AwqLds awq_lds(int K, int MR, int rows) {
  const int TB = K / 512, G = K / 64;
  AwqLds L;
  L.xsl = TB * 64 * MR * 16;
  L.sz = L.xsl + TB * 16 * MR * 4;
  L.trash = L.sz + rows * G * 8;
  L.total = L.trash + 64;
  L.nx = MR * TB * 64;
  L.ns = rows * TB;
  return L;
}
}  // namespace

// Requires K % 512 == 0 (every 16-lane load of a row is whole), K <= 8192,
// N % (4W) == 0 and M <= MR.
// The small-M kernel's body for workgroup `bid`, with its LDS (awq_lds()
// bytes, 16-byte aligned) at lds4; 64 W threads.
template <int MR, int SX, int W>
__device__ __forceinline__ void awq_gemv_body(
    uint4* lds4, int bid, int M, int N, int K, const uint16_t* __restrict__ x, const uint8_t* __restrict__ wc,
    const uint16_t* __restrict__ ws, const uint16_t* __restrict__ wz,
    const uint16_t* __restrict__ bias, uint16_t* __restrict__ y) {
  constexpr int ROWS = 4 * W, NT = 64 * W;
  constexpr int SS = (ROWS * AWQ_TBMAX + NT - 1) / NT;  // scale items per thread
  const int TB = K >> 9, G = K >> 6, rowb = K >> 1;
  const AwqLds L = awq_lds(K, MR, ROWS);
  uint8_t* lds = (uint8_t*)lds4;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int b = lane >> 2, c = lane & 3;
  const int n0 = bid * ROWS;
  const int arow = c % MR;  // A rows past MR only feed D rows that are never read
  const __amdgpu_buffer_rsrc_t xres = __builtin_amdgcn_make_buffer_rsrc((void*)x, (short)0, M * K * 2, kBufDword3);
  const __amdgpu_buffer_rsrc_t wres = __builtin_amdgcn_make_buffer_rsrc((void*)wc, (short)0, N * rowb, kBufDword3);
  const __amdgpu_buffer_rsrc_t sres = __builtin_amdgcn_make_buffer_rsrc((void*)ws, (short)0, N * G * 2, kBufDword3);
  const __amdgpu_buffer_rsrc_t zres = __builtin_amdgcn_make_buffer_rsrc((void*)wz, (short)0, N * G * 2, kBufDword3);

  // Staging loads, issued before the weight loads so that waiting for them
  // (the counter is in order) does not wait for the weights.  x item
  // it = ((m * TB + t) * 16 + chunk-in-block) * 4 + word; scale item
  // q = 8-group block * ROWS + row.  Items past the end read zeros.
  uint4 xw[SX];
#pragma unroll
  for (int j = 0; j < SX; ++j) {
    const int it = tid + j * NT;
    int m = 0, tt = it >> 6;
#pragma unroll
    for (int e = 1; e < MR; ++e)
      if (tt >= TB) { tt -= TB; ++m; }
    const int ch = (tt << 4) + ((it >> 2) & 15);
    const bool ok = it < L.nx && m < M;
    xw[j] = __builtin_bit_cast(
        uint4, __builtin_amdgcn_raw_buffer_load_b128(xres, ok ? (m * K + 32 * ch + 8 * (it & 3)) * 2 : kOut, 0, 0));
  }
  uint4 sr[SS], zr[SS];
#pragma unroll
  for (int j = 0; j < SS; ++j) {
    const int q = tid + j * NT;
    const int off = q < L.ns ? ((n0 + q % ROWS) * G + 8 * (q / ROWS)) * 2 : kOut;
    sr[j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(sres, off, 0, 0));
    zr[j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(zres, off, 0, 0));
  }

  // codes of this lane's chunks in blocks t0 .. t0+AWQ_PT-1 for its rows,
  // block-major so that block u waits only for its own loads
  uint4 cv[AWQ_PT];
  auto load_pass = [&](int t0) {
#pragma unroll
    for (int u = 0; u < AWQ_PT; ++u) {
      const int n = n0 + wave * 4 + c;
      cv[u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                            wres, t0 + u < TB ? n * rowb + 16 * (16 * (t0 + u) + b) : kOut, 0, 0));
    }
  };
  load_pass(0);

  // x as (k, k+4) bf16 pairs in the order the codes are expanded below, and
  // its fp32 sum per 32-channel chunk.  Stores are unconditional (items past
  // the end go to the spare slot).
#pragma unroll
  for (int j = 0; j < SX; ++j) {
    const int it = tid + j * NT;
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
    float sm = dot2bf(w.x, kOnes2, 0.0f);  // fp32 sum of the 8 channels
    sm = dot2bf(w.y, kOnes2, sm);
    sm = dot2bf(w.z, kOnes2, sm);
    sm = dot2bf(w.w, kOnes2, sm);
    // the four words of a chunk are adjacent lanes: sum them with quad DPP moves
    sm += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, sm), 0xB1, 0xF, 0xF, false));
    sm += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, sm), 0x4E, 0xF, 0xF, false));
    *(float*)(lds + (live && i == 0 ? L.xsl + 4 * (((tt << 4) + bb) * MR + m) : L.trash + 16)) = sm;
  }
  // (scale, zero-point + 128) as fp32 pairs
#pragma unroll
  for (int j = 0; j < SS; ++j) {
    const int q = tid + j * NT;
    const bool live = q < L.ns;
    const u32 sw4[4] = {sr[j].x, sr[j].y, sr[j].z, sr[j].w}, zw4[4] = {zr[j].x, zr[j].y, zr[j].z, zr[j].w};
    float4 o[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      o[e] = float4{f16_bits_to_f32(sw4[e] & 0xFFFFu), f16_bits_to_f32(zw4[e] & 0xFFFFu) + 128.0f,
                    f16_bits_to_f32(sw4[e] >> 16), f16_bits_to_f32(zw4[e] >> 16) + 128.0f};
    float4* dst = (float4*)(lds + (live ? L.sz + ((q % ROWS) * G + 8 * (q / ROWS)) * 8 : L.trash));
    const int step = live ? 1 : 0;  // the spare slot takes all four
#pragma unroll
    for (int e = 0; e < 4; ++e) dst[e * step] = o[e];
  }
  __syncthreads();

  const uint4* xl = lds4;
  const float* xsl = (const float*)(lds + L.xsl);
  const float2* szl = (const float2*)(lds + L.sz);
  const u32 kMask = in_vgpr(0x000F000Fu), kBf128 = in_vgpr(0x43004300u);

  float acc[MR];
#pragma unroll
  for (int v = 0; v < MR; ++v) acc[v] = 0.0f;

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
      {
        const int r = wave * 4 + c;
        const float2 sz = szl[r * G + 8 * t + (b >> 1)];
        const u32 d4[4] = {cv[u].x, cv[u].y, cv[u].z, cv[u].w};
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
        for (int v = 0; v < MR; ++v) acc[v] = fmaf(sz.x, fmaf(-sz.y, xs[v], d[v]), acc[v]);
      }
    }
    t0 += AWQ_PT;
    if (t0 >= TB) break;
    load_pass(t0);
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
    const int n = n0 + wave * 4 + c;
    const float bv = bias ? bf16_bits_to_f32(bias[n]) : 0.0f;
#pragma unroll
    for (int v = 0; v < MR; ++v)
      if (v < M) y[(size_t)v * N + n] = (uint16_t)f32_to_bf16_bits(acc[v] + bv);
  }
}

}  // namespace svdq
