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
#include <type_traits>

#include "common.h"
#include "launch.h"

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
template <int MR, int SX, int W>
__global__ __launch_bounds__(64 * W) void awq_gemv_kernel(
    int M, int N, int K, const uint16_t* __restrict__ x, const uint8_t* __restrict__ wc,
    const uint16_t* __restrict__ ws, const uint16_t* __restrict__ wz,
    const uint16_t* __restrict__ bias, uint16_t* __restrict__ y) {
  constexpr int ROWS = 4 * W, NT = 64 * W;
  constexpr int SS = (ROWS * AWQ_TBMAX + NT - 1) / NT;  // scale items per thread
  extern __shared__ __align__(16) uint4 lds4[];
  const int TB = K >> 9, G = K >> 6, rowb = K >> 1;
  const AwqLds L = awq_lds(K, MR, ROWS);
  uint8_t* lds = (uint8_t*)lds4;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int b = lane >> 2, c = lane & 3;
  const int n0 = blockIdx.x * ROWS;
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

// Other shapes (4 < M <= 64, or a K the small kernel does not take):
//   D[m][n] = sum_{k in g} x[m,k] * (128 + q[n,k]) per 64-channel group on the
//   bf16 matrix cores (both operands exact in bf16), then in fp32
//   acc[m][n] += s[n,g] * (D[m][n] - (z[n,g] + 128) * xsum[m,g]).
// Workgroup: 64 weight rows x 64 activation rows (rows past M read as zero);
// wave w owns the 32x32 block (m half w&1, n half (w>>1)&1).  The matrix-core A
// operand is x (rows m) and B the weight tile (columns n), so each lane holds
// one column n: its scale and zero-point are per-lane scalars and each store
// of the 32 lanes covers 64 contiguous bytes of a Y row.  Eight waves: waves
// 0-3 take the first 64-channel group of every stage and waves 4-7 the
// second, so two waves share each SIMD; their partial sums meet in LDS at
// the end (fixed order).  Stages of two groups are double buffered in LDS;
// x, codes, scales and zero-points are loaded two stages ahead into two
// register sets (branch-free buffer loads).  Within each 8-channel block both operands take the channel
// order (k0,k4) (k1,k5) (k2,k6) (k3,k7), which is the order the AND-OR code
// expansion produces.
namespace {
constexpr int AG_ROW = 136;  // bf16 per LDS row: two 64-channel groups + 8 padding
struct AwqGemmLds {
  uint16_t x[2][64 * AG_ROW];   // x pairs, per buffer
  uint16_t w[2][64 * AG_ROW];   // 128 + q as bf16, per buffer
  float xs[2][2][64];           // [buffer][group][m] sum of x over the group
  float sc[2][2][64];           // [buffer][group][n] scale
  float zp[2][2][64];           // [buffer][group][n] zero-point + 128
};
}  // namespace

__global__ __launch_bounds__(512) void awq_gemm_mfma_kernel(
    int M, int N, int K, const uint16_t* __restrict__ x, const uint8_t* __restrict__ wc,
    const uint16_t* __restrict__ ws, const uint16_t* __restrict__ wz,
    const uint16_t* __restrict__ bias, uint16_t* __restrict__ y) {
  extern __shared__ __align__(16) uint8_t awq_smem[];
  AwqGemmLds& L = *(AwqGemmLds*)awq_smem;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int n0 = blockIdx.x * 64;
  const int G = K >> 6, rowb = K >> 1, stages = (G + 1) >> 1;
  // waves 0-3 take the first group of every stage, waves 4-7 the second
  const int half = wave >> 2;
  const int bm = (wave & 1) * 32, bn = ((wave >> 1) & 1) * 32;
  const int lr = lane & 31, lh = lane >> 5;
  const __amdgpu_buffer_rsrc_t xres = __builtin_amdgcn_make_buffer_rsrc((void*)x, (short)0, M * K * 2, kBufDword3);
  const __amdgpu_buffer_rsrc_t wres = __builtin_amdgcn_make_buffer_rsrc((void*)wc, (short)0, N * rowb, kBufDword3);
  const __amdgpu_buffer_rsrc_t sres = __builtin_amdgcn_make_buffer_rsrc((void*)ws, (short)0, N * G * 2, kBufDword3);
  const __amdgpu_buffer_rsrc_t zres = __builtin_amdgcn_make_buffer_rsrc((void*)wz, (short)0, N * G * 2, kBufDword3);

  // staging roles: x chunk c = tid + 512 r (r < 2) -> row c/16, 8-channel block
  // c%16; threads < 256: codes of row tid/4, 32 codes (tid%4); threads >= 256:
  // scale (t < 384) or zero-point of row t%64, group (t/64)%2
  // Two register sets: the loads for stage st + 2 are issued at the start of
  // stage st and expanded into LDS at the end of stage st + 1; loads past the
  // last stage read zeros (offset beyond the buffer), and scheduling barriers
  // keep the expansion at the end of a stage (the compiler would otherwise
  // hoist it up to the loads and wait for them at once).
  uint4 xv[2][2], wv[2];
  u32 szv[2];
  const bool is_w = tid < 256;
  auto gload = [&](int st, auto setc) {
    constexpr int set = decltype(setc)::value;
    const bool live = st < stages;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int c = tid + 512 * r, row = c >> 4, blk = c & 15;
      const bool ok = live && row < M && 2 * st + (blk >> 3) < G;
      xv[set][r] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                                 xres, ok ? (row * K + 128 * st + 8 * blk) * 2 : kOut, 0, 0));
    }
    if (is_w) {  // wave-uniform
      const int row = tid >> 2, part = tid & 3;
      const bool ok = live && 2 * st + (part >> 1) < G;
      wv[set] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                              wres, ok ? (n0 + row) * rowb + 64 * st + 16 * part : kOut, 0, 0));
    } else {
      const int row = tid & 63, g = 2 * st + ((tid >> 6) & 1);
      const int off = live && g < G ? ((n0 + row) * G + g) * 2 : kOut;
      szv[set] = tid < 384 ? __builtin_amdgcn_raw_buffer_load_b16(sres, off, 0, 0)
                           : __builtin_amdgcn_raw_buffer_load_b16(zres, off, 0, 0);
    }
  };
  auto sstore = [&](int buf, auto setc) {
    constexpr int set = decltype(setc)::value;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int c = tid + 512 * r, row = c >> 4, blk = c & 15;
      const uint4 v = xv[set][r];
      *(uint4*)&L.x[buf][row * AG_ROW + 8 * blk] =
          uint4{__builtin_amdgcn_perm(v.z, v.x, 0x05040100u), __builtin_amdgcn_perm(v.z, v.x, 0x07060302u),
                __builtin_amdgcn_perm(v.w, v.y, 0x05040100u), __builtin_amdgcn_perm(v.w, v.y, 0x07060302u)};
      // fp32 sum of the 8 channels: pairs of bf16 times (1, 1) on v_dot2_f32_bf16
      float sm = dot2bf(v.x, kOnes2, 0.0f);
      sm = dot2bf(v.y, kOnes2, sm);
      sm = dot2bf(v.z, kOnes2, sm);
      sm = dot2bf(v.w, kOnes2, sm);
      // the 8 blocks of a group are 8 adjacent lanes: quad DPP, then the lane 4 above
      sm += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, sm), 0xB1, 0xF, 0xF, false));
      sm += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, sm), 0x4E, 0xF, 0xF, false));
      sm += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, sm), 0x104, 0xF, 0xF, false));
      if ((blk & 7) == 0) L.xs[buf][blk >> 3][row] = sm;
    }
    if (is_w) {
      const int row = tid >> 2, part = tid & 3;
      const u32 d4[4] = {wv[set].x, wv[set].y, wv[set].z, wv[set].w};
      u32 o[16];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const u32 d = d4[i];
        o[4 * i + 0] = (d & 0x000F000Fu) | 0x43004300u;          // (k0, k4)
        o[4 * i + 1] = ((d >> 4) & 0x000F000Fu) | 0x43004300u;   // (k1, k5)
        o[4 * i + 2] = ((d >> 8) & 0x000F000Fu) | 0x43004300u;   // (k2, k6)
        o[4 * i + 3] = ((d >> 12) & 0x000F000Fu) | 0x43004300u;  // (k3, k7)
      }
      uint16_t* dst = &L.w[buf][row * AG_ROW + 32 * part];
#pragma unroll
      for (int i = 0; i < 4; ++i) *(uint4*)(dst + 8 * i) = uint4{o[4 * i], o[4 * i + 1], o[4 * i + 2], o[4 * i + 3]};
    } else {
      const int row = tid & 63, g = (tid >> 6) & 1;
      const float v = f16_bits_to_f32(szv[set]);
      if (tid < 384) L.sc[buf][g][row] = v;
      else L.zp[buf][g][row] = v + 128.0f;
    }
  };

  v16f acc;
#pragma unroll
  for (int v = 0; v < 16; ++v) acc[v] = 0.0f;

  gload(0, std::integral_constant<int, 0>{});
  gload(1, std::integral_constant<int, 1>{});
  sstore(0, std::integral_constant<int, 0>{});
  __syncthreads();
  auto stage = [&](int st, auto setc) __attribute__((always_inline)) {
    constexpr int set = decltype(setc)::value;
    const int buf = st & 1;
    gload(st + 2, setc);
    __builtin_amdgcn_sched_barrier(0);
    if (2 * st + half < G) {  // wave-uniform: a last stage may hold one group
      const int gg = half;
      v16f d;
#pragma unroll
      for (int v = 0; v < 16; ++v) d[v] = 0.0f;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const v8bf a = *(const v8bf*)&L.x[buf][(bm + lr) * AG_ROW + 64 * gg + 16 * kk + 8 * lh];
        const v8bf b = *(const v8bf*)&L.w[buf][(bn + lr) * AG_ROW + 64 * gg + 16 * kk + 8 * lh];
        d = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, d, 0, 0, 0);
      }
      const float sc = L.sc[buf][gg][bn + lr], zp = L.zp[buf][gg][bn + lr];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 xs4 = *(const float4*)&L.xs[buf][gg][bm + 8 * q + 4 * lh];
        const float xs[4] = {xs4.x, xs4.y, xs4.z, xs4.w};
#pragma unroll
        for (int v = 0; v < 4; ++v)
          acc[4 * q + v] = fmaf(sc, fmaf(-zp, xs[v], d[4 * q + v]), acc[4 * q + v]);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    // past the last stage this fills the idle buffer, which nothing reads
    sstore(buf ^ 1, std::integral_constant<int, set ^ 1>{});
    __syncthreads();
  };
  {
    int st = 0;
    for (; st + 1 < stages; st += 2) {
      stage(st, std::integral_constant<int, 0>{});
      stage(st + 1, std::integral_constant<int, 1>{});
    }
    if (st < stages) stage(st, std::integral_constant<int, 0>{});
  }

  // the second half's partial sums go through LDS (the staging space is free now)
  float* red = (float*)awq_smem;  // [4 blocks][64 lanes][16]
  const int blkid = wave & 3;
  if (half == 1) {
#pragma unroll
    for (int v = 0; v < 16; v += 4)
      *(float4*)&red[(blkid * 64 + lane) * 16 + v] = float4{acc[v], acc[v + 1], acc[v + 2], acc[v + 3]};
  }
  __syncthreads();
  if (half == 0) {
#pragma unroll
    for (int v = 0; v < 16; v += 4) {
      const float4 o = *(const float4*)&red[(blkid * 64 + lane) * 16 + v];
      acc[v] += o.x; acc[v + 1] += o.y; acc[v + 2] += o.z; acc[v + 3] += o.w;
    }
    const int n = n0 + bn + lr;
    const float bv = bias ? bf16_bits_to_f32(bias[n]) : 0.0f;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int m = bm + 8 * (v >> 2) + 4 * lh + (v & 3);
      if (m < M) y[(size_t)m * N + n] = (uint16_t)f32_to_bf16_bits(acc[v] + bv);
    }
  }
}

using AwqKern = void (*)(int, int, int, const uint16_t*, const uint8_t*, const uint16_t*, const uint16_t*,
                         const uint16_t*, uint16_t*);
template <int W>
AwqKern awq_small_kernel(int mr_idx, int sx_idx) {
  static const AwqKern table[3][4] = {
      {awq_gemv_kernel<1, 1, W>, awq_gemv_kernel<1, 2, W>, awq_gemv_kernel<1, 4, W>, awq_gemv_kernel<1, 8, W>},
      {awq_gemv_kernel<2, 1, W>, awq_gemv_kernel<2, 2, W>, awq_gemv_kernel<2, 4, W>, awq_gemv_kernel<2, 8, W>},
      {awq_gemv_kernel<4, 1, W>, awq_gemv_kernel<4, 2, W>, awq_gemv_kernel<4, 4, W>, awq_gemv_kernel<4, 8, W>}};
  return table[mr_idx][sx_idx];
}

hipError_t launch_awq(const AwqArgs& a, hipStream_t st) {
  const int M = (int)a.M, N = (int)a.N, K = (int)a.K;
  const int MR = M <= 1 ? 1 : M <= 2 ? 2 : 4;
  // Small-M kernel: of the wave counts (8, 6, 4 waves of 4 rows) that fit the
  // shape, the one whose workgroups fill the 256 CUs most evenly (smallest
  // ratio of rounds started, ceil(workgroups / 256), to rounds of work).
  int W = 0, si = 0;
  long best = 0, best_den = 1;  // compare ceil(wg/256)/(wg/256) as fractions
  if (M <= 4 && K % 512 == 0 && K / 512 <= AWQ_TBMAX) {
    for (int w : {8, 6, 4}) {
      if (N % (4 * w) != 0) continue;
      const AwqLds L = awq_lds(K, MR, 4 * w);
      const int items = (L.nx + 64 * w - 1) / (64 * w);  // x staging items per thread
      if (L.total > 64 * 1024 || items > 8) continue;
      const long wg = N / (4 * w), rounds = (wg + 255) / 256;
      // rounds * 256 / wg < best / best_den
      if (W == 0 || rounds * 256 * best_den < best * wg) {
        W = w; si = items; best = rounds * 256; best_den = wg;
      }
    }
  }
  if (W) {
    const AwqLds L = awq_lds(K, MR, 4 * W);
    const int mi = MR == 1 ? 0 : MR == 2 ? 1 : 2;
    const int sidx = si <= 1 ? 0 : si <= 2 ? 1 : si <= 4 ? 2 : 3;
    const AwqKern k = W == 8 ? awq_small_kernel<8>(mi, sidx) : W == 6 ? awq_small_kernel<6>(mi, sidx)
                                                                      : awq_small_kernel<4>(mi, sidx);
    hipLaunchKernelGGL(k, dim3(N / (4 * W)), dim3(64 * W), L.total, st,
                       M, N, K, (const uint16_t*)a.x, (const uint8_t*)a.w_codes, (const uint16_t*)a.w_scales,
                       (const uint16_t*)a.w_zeros, (const uint16_t*)a.bias, (uint16_t*)a.y);
  } else {
    const hipError_t e = hipFuncSetAttribute((const void*)awq_gemm_mfma_kernel,
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)sizeof(AwqGemmLds));
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(awq_gemm_mfma_kernel, dim3(N / 64), dim3(512), sizeof(AwqGemmLds), st, M, N, K,
                       (const uint16_t*)a.x, (const uint8_t*)a.w_codes, (const uint16_t*)a.w_scales,
                       (const uint16_t*)a.w_zeros, (const uint16_t*)a.bias, (uint16_t*)a.y);
  }
  return hipGetLastError();
}

}  // namespace svdq
