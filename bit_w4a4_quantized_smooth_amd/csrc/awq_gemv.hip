// AWQ W4A16 linear ("Nunchaku Lite", "Supported quantization types":
// awq_w4a16, int4 weight-only, group 64; blog "Nunchaku 4-bit inference in
// Diffusers", "Introducing Nunchaku Lite": memory-bound modulation
// projections):
//   y[m,n] = sum_g s[n,g] * ( sum_{k in g} x[m,k] * q[n,k]  -  z[n,g] * sum_{k in g} x[m,k] ) + bias[n]
// which equals sum_k x * (q - z) * s (the weight dequantized per group).
//
// Three kernels:
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
//  * other M with K % 512 == 0: one workgroup per CU, the weights streamed
//    through an LDS ring by buffer loads to LDS (awq_stream_kernel).
//  * K % 512 != 0: a 64x64-tile matrix-core kernel with LDS staging
//    (awq_gemm_mfma_kernel).
#include <type_traits>

#include "awq_small.h"
#include "common.h"
#include "launch.h"

namespace svdq {

// Requires K % 512 == 0 (every 16-lane load of a row is whole), K <= 8192,
// N % (4W) == 0 and M <= MR.
template <int MR, int SX, int W>
__global__ __launch_bounds__(64 * W) void awq_gemv_kernel(
    int M, int N, int K, const uint16_t* __restrict__ x, const uint8_t* __restrict__ wc,
    const uint16_t* __restrict__ ws, const uint16_t* __restrict__ wz,
    const uint16_t* __restrict__ bias, uint16_t* __restrict__ y) {
  extern __shared__ __align__(16) uint4 lds4[];
  awq_gemv_body<MR, SX, W>(lds4, (int)blockIdx.x, M, N, K, x, wc, ws, wz, bias, y);
}

// K % 512 != 0 (any M <= 64):
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

// ---- M > 4 (and K the small kernel does not take): weights streamed through LDS
// y = x . W^T with W = (q - z) s per (row, 64-group).  The weight rows are cut
// into units of 16; workgroup w (one per CU) owns a contiguous run of units and
// takes them in batches of up to 5.  K is cut into chunks of 8 groups (512
// channels); the eight waves work through the chunks in lockstep, wave i on
// group i of each chunk, so every wave holds partial sums for all of the
// batch's outputs and the eight are added in LDS at the end.
//
// Weight codes, scales and zero-points of a chunk are copied from memory
// straight into an LDS ring of 6 chunks by buffer loads to LDS: 256
// contiguous bytes of each weight row per chunk, and 16 bytes (8 fp16) of each
// scale and zero-point row.  No register holds them in flight, so a CU keeps
// up to five chunks (120 KB at 80 rows) of weights in flight.  The 16-byte
// columns of a row sit XOR-swizzled by the row's low four bits, so the 16
// rows a matrix-core operand reads fall in distinct banks.  x goes straight
// from memory (it stays in L2: every CU reads all of it) into registers two
// chunks ahead.  Each workgroup starts at its own chunk (rotation by the
// workgroup index), so the CUs do not all read the same x lines at once.
//
// Per group, on v_mfma_f32_16x16x32_bf16:
//   A = x, 16 rows per m-block; lane (row l16, quarter lg) holds the channels
//       64g + 16lg + 8j + t of k-step j (t = 0..7): 32 contiguous bytes of x
//   B = 128 + q as bf16 (nibble | 0x4300, exact), the same channels of its row
// so two products give P'[m][n] = sum x (128 + q) over the group, and the
// same products against a ones operand give xs[m] = sum x, in the same
// register layout as P' (each lane holds the rows 4 lg + v).  Then
//   acc += s * (P' - (128 + z) xs),
// two FMAs per output and group; the difference is taken per group, before
// any scaling.
namespace {
constexpr int AS_NT = 512, AS_UB = 5, AS_D = 6;
// 1 KB wave-instructions per chunk and wave: codes of 16 UB rows x 256 B
// (4 UB instructions), then scales and zero-points for rows 0-63 and 64-127
// (4 instructions), spread over the eight waves; the remainder up to a
// multiple of 8 are loads past the end that only write zeros.
__host__ __device__ constexpr int as_niw(int UB) { return (4 * UB + 4 + 7) / 8; }
__host__ __device__ constexpr int as_slot(int UB) { return as_niw(UB) * 8 * 1024; }
__host__ __device__ constexpr size_t as_lds_bytes(int UB, int MB) {
  // the ring, reused at the end for two [8 waves][16 MB][16] fp32 reduction buffers
  return (size_t)AS_D * as_slot(UB) > (size_t)2 * 8 * MB * 256 * 4 ? (size_t)AS_D * as_slot(UB)
                                                                    : (size_t)2 * 8 * MB * 256 * 4;
}
typedef __attribute__((address_space(3))) void as_lds_void;
typedef __attribute__((address_space(3))) const uint8_t as_lds_u8;

__device__ __forceinline__ uint4 as_expand8(u32 d) {  // 8 codes -> 8 bf16 (128 + q), natural channel order
  const u32 sh = d >> 4;
  const u32 m = in_vgpr(0x000F000Fu), o = in_vgpr(0x43004300u);
  return uint4{(__builtin_amdgcn_perm(sh, d, 0x0C040C00u) & m) | o, (__builtin_amdgcn_perm(sh, d, 0x0C050C01u) & m) | o,
               (__builtin_amdgcn_perm(sh, d, 0x0C060C02u) & m) | o, (__builtin_amdgcn_perm(sh, d, 0x0C070C03u) & m) | o};
}

// The LDS reads of one chunk step (per unit: 8 code bytes, the scale and the
// zero-point), issued together and waited for in the same statement.  Reads
// the compiler sees after a copy to LDS make it wait for every copy in flight
// (it cannot tell which slot a copy wrote), which would drain the ring.
// a: byte address of unit 0's codes (unit u: + 4096 u); t: of unit 0's scale
// (unit u < 4: + 256 u, unit 4: + 2048; the zero-point 1024 bytes above).
template <int UB> struct SlotReads { uint2 c[UB]; u32 s[UB], z[UB]; };
#define AS_RD3(ci, si, zi, oc, os, oz)                                                         \
  "ds_read_b64 %" #ci ", %[a] offset:" #oc "\n\tds_read_u16 %" #si ", %[t] offset:" #os "\n\t" \
  "ds_read_u16 %" #zi ", %[t] offset:" #oz "\n\t"
#define AS_U0(c, s, z) AS_RD3(c, s, z, 0, 0, 1024)
#define AS_U1(c, s, z) AS_RD3(c, s, z, 4096, 256, 1280)
#define AS_U2(c, s, z) AS_RD3(c, s, z, 8192, 512, 1536)
#define AS_U3(c, s, z) AS_RD3(c, s, z, 12288, 768, 1792)
#define AS_U4(c, s, z) AS_RD3(c, s, z, 16384, 2048, 3072)
template <int UB>
__device__ __forceinline__ SlotReads<UB> as_slot_reads(u32 a, u32 t) {
  SlotReads<UB> r;
  if constexpr (UB == 1) {
    asm volatile(AS_U0(0, 1, 2) "s_waitcnt lgkmcnt(0)"
                 : "=&v"(r.c[0]), "=&v"(r.s[0]), "=&v"(r.z[0]) : [a] "v"(a), [t] "v"(t));
  } else if constexpr (UB == 2) {
    asm volatile(AS_U0(0, 2, 4) AS_U1(1, 3, 5) "s_waitcnt lgkmcnt(0)"
                 : "=&v"(r.c[0]), "=&v"(r.c[1]), "=&v"(r.s[0]), "=&v"(r.s[1]), "=&v"(r.z[0]), "=&v"(r.z[1])
                 : [a] "v"(a), [t] "v"(t));
  } else if constexpr (UB == 3) {
    asm volatile(AS_U0(0, 3, 6) AS_U1(1, 4, 7) AS_U2(2, 5, 8) "s_waitcnt lgkmcnt(0)"
                 : "=&v"(r.c[0]), "=&v"(r.c[1]), "=&v"(r.c[2]), "=&v"(r.s[0]), "=&v"(r.s[1]), "=&v"(r.s[2]),
                   "=&v"(r.z[0]), "=&v"(r.z[1]), "=&v"(r.z[2])
                 : [a] "v"(a), [t] "v"(t));
  } else if constexpr (UB == 4) {
    asm volatile(AS_U0(0, 4, 8) AS_U1(1, 5, 9) AS_U2(2, 6, 10) AS_U3(3, 7, 11) "s_waitcnt lgkmcnt(0)"
                 : "=&v"(r.c[0]), "=&v"(r.c[1]), "=&v"(r.c[2]), "=&v"(r.c[3]), "=&v"(r.s[0]), "=&v"(r.s[1]),
                   "=&v"(r.s[2]), "=&v"(r.s[3]), "=&v"(r.z[0]), "=&v"(r.z[1]), "=&v"(r.z[2]), "=&v"(r.z[3])
                 : [a] "v"(a), [t] "v"(t));
  } else {
    static_assert(UB == 5, "up to 5 units");
    asm volatile(AS_U0(0, 5, 10) AS_U1(1, 6, 11) AS_U2(2, 7, 12) AS_U3(3, 8, 13) AS_U4(4, 9, 14)
                 "s_waitcnt lgkmcnt(0)"
                 : "=&v"(r.c[0]), "=&v"(r.c[1]), "=&v"(r.c[2]), "=&v"(r.c[3]), "=&v"(r.c[4]), "=&v"(r.s[0]),
                   "=&v"(r.s[1]), "=&v"(r.s[2]), "=&v"(r.s[3]), "=&v"(r.s[4]), "=&v"(r.z[0]), "=&v"(r.z[1]),
                   "=&v"(r.z[2]), "=&v"(r.z[3]), "=&v"(r.z[4])
                 : [a] "v"(a), [t] "v"(t));
  }
  return r;
}
#undef AS_U0
#undef AS_U1
#undef AS_U2
#undef AS_U3
#undef AS_U4
#undef AS_RD3
}  // namespace

// Requires K % 512 == 0 and N % 16 == 0.
template <int UB, int MB>
__global__ __launch_bounds__(AS_NT) void awq_stream_kernel(
    int M, int N, int K, const uint16_t* __restrict__ x, const uint8_t* __restrict__ wc,
    const uint16_t* __restrict__ ws, const uint16_t* __restrict__ wz,
    const uint16_t* __restrict__ bias, uint16_t* __restrict__ y) {
  extern __shared__ __align__(16) uint8_t as_lds[];
  constexpr int NIW = as_niw(UB), SLOT = as_slot(UB);
  constexpr int TAB = 4 * UB * 1024;  // offset of the scale/zero-point tables in a slot
  const int G = K >> 6, NC = G >> 3, rowb = K >> 1;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, lg = lane >> 4;
  const int units = N >> 4;
  const int u0 = (int)(((long)blockIdx.x * units) / gridDim.x), u1 = (int)(((long)(blockIdx.x + 1) * units) / gridDim.x);
  const int rot = (int)(blockIdx.x % (unsigned)NC);

  const __amdgpu_buffer_rsrc_t xres = __builtin_amdgcn_make_buffer_rsrc((void*)x, (short)0, M * K * 2, kBufDword3);
  const __amdgpu_buffer_rsrc_t wres = __builtin_amdgcn_make_buffer_rsrc((void*)wc, (short)0, N * rowb, kBufDword3);
  const __amdgpu_buffer_rsrc_t sres = __builtin_amdgcn_make_buffer_rsrc((void*)ws, (short)0, N * G * 2, kBufDword3);
  const __amdgpu_buffer_rsrc_t zres = __builtin_amdgcn_make_buffer_rsrc((void*)wz, (short)0, N * G * 2, kBufDword3);
  const v8bf ones = __builtin_bit_cast(v8bf, uint4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u});
  const v4f zero4 = {0.f, 0.f, 0.f, 0.f};

  for (int ub = u0; ub < u1; ub += UB) {
    const int rows = 16 * (u1 - ub < UB ? u1 - ub : UB);  // weight rows of this batch
    const int nu = rows >> 4;
    const int n0 = ub * 16;
    // chunk c of the loop is chunk (c + rot) mod NC of K
    auto chunk = [&](int c) { return c + rot >= NC ? c + rot - NC : c + rot; };
    // this wave's share of the copies of loop chunk c into its ring slot; past
    // the last chunk the same loads read nothing and fill the slot with zeros
    // (always issued, so that the memory counter advances the same way each step)
    auto dma = [&](int c) __attribute__((always_inline)) {
      const bool live = c < NC;
      const int cc = chunk(live ? c : 0);
      uint8_t* slot = as_lds + (c % AS_D) * SLOT;
#pragma unroll
      for (int i = 0; i < NIW; ++i) {
        const int j = wave + 8 * i;  // instruction of the chunk, wave-uniform
        as_lds_void* dst = (as_lds_void*)(slot + 1024 * j);
        if (j < 4 * UB) {  // codes: rows 4j .. 4j+3, lane -> (row, swizzled 16-byte column)
          const int r = 4 * j + (lane >> 4), col = (lane & 15) ^ (r & 15);
          const int off = live && r < rows ? (n0 + r) * rowb + 256 * cc + 16 * col : kOut;
          __builtin_amdgcn_raw_ptr_buffer_load_lds(wres, dst, 16, off, 0, 0, 0);
        } else if (j < 4 * UB + 4) {  // scales (even) / zero-points (odd) of rows 64 t' + lane
          const int t = j - 4 * UB, r = 64 * (t >> 1) + lane;
          const int off = live && r < rows ? ((n0 + r) * G + 8 * cc) * 2 : kOut;
          if (t & 1) __builtin_amdgcn_raw_ptr_buffer_load_lds(zres, dst, 16, off, 0, 0, 0);
          else __builtin_amdgcn_raw_ptr_buffer_load_lds(sres, dst, 16, off, 0, 0, 0);
        } else {
          __builtin_amdgcn_raw_ptr_buffer_load_lds(wres, dst, 16, kOut, 0, 0, 0);
        }
      }
    };
    uint4 xv[2][MB][2];
    auto xload = [&](int c, auto setc) __attribute__((always_inline)) {
      constexpr int S = decltype(setc)::value;
      const int g = 8 * chunk(c < NC ? c : 0) + wave;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const int off = c < NC ? ((16 * mb + l16) * K + 64 * g + 16 * lg) * 2 : kOut;
        xv[S][mb][0] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(xres, off, 0, 0));
        xv[S][mb][1] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(xres, c < NC ? off + 16 : kOut, 0, 0));
      }
    };
    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;

    v4f acc[UB][MB];
#pragma unroll
    for (int u = 0; u < UB; ++u)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) acc[u][mb] = zero4;

    auto compute = [&](int c, auto setc) __attribute__((always_inline)) {
      constexpr int S = decltype(setc)::value;
      const uint8_t* slot = as_lds + (c % AS_D) * SLOT;
      v8bf xa[MB][2];
      v4f xs[MB];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        xa[mb][0] = __builtin_bit_cast(v8bf, xv[S][mb][0]);
        xa[mb][1] = __builtin_bit_cast(v8bf, xv[S][mb][1]);
        xs[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[mb][0], ones, zero4, 0, 0, 0);
        xs[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[mb][1], ones, xs[mb], 0, 0, 0);
      }
      // unit 0's 32-bit LDS addresses in the slot (row l16); the other units
      // are constant offsets (units past nu read rows the copies zero-filled)
      const u32 sb = (u32)(uintptr_t)(const as_lds_u8*)slot;
      const SlotReads<UB> rd = as_slot_reads<UB>(sb + l16 * 256 + 16 * ((2 * wave + (lg >> 1)) ^ l16) + 8 * (lg & 1),
                                                 sb + TAB + 16 * l16 + 2 * wave);
#pragma unroll
      for (int u = 0; u < UB; ++u) {
        if (u < nu) {  // wave-uniform
          const float sc = f16_bits_to_f32(rd.s[u] & 0xFFFFu);
          const float zz = f16_bits_to_f32(rd.z[u] & 0xFFFFu) + 128.0f;
          const v8bf b0 = __builtin_bit_cast(v8bf, as_expand8(rd.c[u].x));
          const v8bf b1 = __builtin_bit_cast(v8bf, as_expand8(rd.c[u].y));
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) {
            v4f p = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[mb][0], b0, zero4, 0, 0, 0);
            p = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[mb][1], b1, p, 0, 0, 0);
#pragma unroll
            for (int v = 0; v < 4; ++v) acc[u][mb][v] = fmaf(sc, fmaf(-zz, xs[mb][v], p[v]), acc[u][mb][v]);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    };

    // Issue order per loop chunk c: [copies of chunk c + D - 1] [compute c]
    // [x of chunk c + 2]; the prologue issues what chunks -2 and -1 would
    // have, so that at the top of chunk c the memory operations issued after
    // x of chunk c are exactly the copies of chunk c + D - 2 and x of c + 1.
    // Waiting for x of chunk c also covers the copies of chunk c (issued at
    // least one chunk earlier, as D >= 4; the memory counter is in order).
    static_assert(AS_D >= 4, "the wait for x covers the copies only when D >= 4");
    for (int c = 0; c <= AS_D - 3; ++c) dma(c);
    xload(0, S0{});
    dma(AS_D - 2);
    xload(1, S1{});
    auto step = [&](int c, auto setc) __attribute__((always_inline)) {
      {
        constexpr int n = NIW + 2 * MB;
        __builtin_amdgcn_s_waitcnt((n & 0xF) | ((n >> 4) << 14) | 0x0070 | 0x0F00);
      }
      // Every wave's copies of chunk c have landed and every wave's reads of
      // slot (c - 1) % D are done (waited inside the read statement): a plain
      // barrier suffices.  __syncthreads() would add a release fence, which
      // waits for all copies in flight, the newest included.
      asm volatile("s_barrier" ::: "memory");
      dma(c + AS_D - 1);
      compute(c, setc);
      xload(c + 2, setc);
    };
    int c = 0;
    for (; c + 1 < NC; c += 2) {
      step(c, S0{});
      step(c + 1, S1{});
    }
    if (c < NC) step(c, S0{});

    // the eight waves' partial sums, one unit at a time, through two
    // alternating LDS buffers [8 waves][16 MB rows][16 columns]
    __syncthreads();  // the ring is free
#pragma unroll
    for (int u = 0; u < UB; ++u) {
      if (u < nu) {  // uniform over the workgroup
        float* red = (float*)as_lds + (u & 1) * (8 * MB * 256);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int v = 0; v < 4; ++v) red[(wave * 16 * MB + 16 * mb + 4 * lg + v) * 16 + l16] = acc[u][mb][v];
        __syncthreads();
        for (int o = tid; o < 256 * MB; o += AS_NT) {
          const int m = o >> 4, nn = o & 15;
          float t = 0.0f;
#pragma unroll
          for (int w = 0; w < 8; ++w) t += red[(w * 16 * MB + m) * 16 + nn];  // fixed order
          const int n = n0 + 16 * u + nn;
          if (m < M) y[(size_t)m * N + n] = (uint16_t)f32_to_bf16_bits(t + (bias ? bf16_bits_to_f32(bias[n]) : 0.0f));
        }
      }
    }
    __syncthreads();  // the next batch's copies overwrite the reduction buffers
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
  } else if (K % 512 == 0) {
    // one workgroup per CU over 16-row units of the weight, in batches of up to 5
    const int units = N / 16;
    const int nwg = units < device_cu_count() ? units : device_cu_count();
    const int per = (units + nwg - 1) / nwg;
    const int MBv = M <= 16 ? 1 : M <= 32 ? 2 : M <= 48 ? 3 : 4;
    // four m-blocks hold 16 accumulators per unit: batches of at most 3 units
    // keep a wave within its 256 registers
    const int ubmax = MBv == 4 ? 3 : AS_UB, nb = (per + ubmax - 1) / ubmax;
    const int UBv = (per + nb - 1) / nb;
    using StreamK = void (*)(int, int, int, const uint16_t*, const uint8_t*, const uint16_t*, const uint16_t*,
                             const uint16_t*, uint16_t*);
    static const StreamK table[AS_UB][4] = {
        {awq_stream_kernel<1, 1>, awq_stream_kernel<1, 2>, awq_stream_kernel<1, 3>, awq_stream_kernel<1, 4>},
        {awq_stream_kernel<2, 1>, awq_stream_kernel<2, 2>, awq_stream_kernel<2, 3>, awq_stream_kernel<2, 4>},
        {awq_stream_kernel<3, 1>, awq_stream_kernel<3, 2>, awq_stream_kernel<3, 3>, awq_stream_kernel<3, 4>},
        {awq_stream_kernel<4, 1>, awq_stream_kernel<4, 2>, awq_stream_kernel<4, 3>, awq_stream_kernel<4, 4>},
        {awq_stream_kernel<5, 1>, awq_stream_kernel<5, 2>, awq_stream_kernel<5, 3>, awq_stream_kernel<5, 4>}};
    static const size_t lds_of[AS_UB][4] = {
        {as_lds_bytes(1, 1), as_lds_bytes(1, 2), as_lds_bytes(1, 3), as_lds_bytes(1, 4)},
        {as_lds_bytes(2, 1), as_lds_bytes(2, 2), as_lds_bytes(2, 3), as_lds_bytes(2, 4)},
        {as_lds_bytes(3, 1), as_lds_bytes(3, 2), as_lds_bytes(3, 3), as_lds_bytes(3, 4)},
        {as_lds_bytes(4, 1), as_lds_bytes(4, 2), as_lds_bytes(4, 3), as_lds_bytes(4, 4)},
        {as_lds_bytes(5, 1), as_lds_bytes(5, 2), as_lds_bytes(5, 3), as_lds_bytes(5, 4)}};
    const StreamK kf = table[UBv - 1][MBv - 1];
    const size_t lds = lds_of[UBv - 1][MBv - 1];
    const hipError_t e = hipFuncSetAttribute((const void*)kf, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kf, dim3(nwg), dim3(AS_NT), lds, st, M, N, K, (const uint16_t*)a.x, (const uint8_t*)a.w_codes,
                       (const uint16_t*)a.w_scales, (const uint16_t*)a.w_zeros, (const uint16_t*)a.bias, (uint16_t*)a.y);
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
