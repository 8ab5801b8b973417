// W4A4 NVFP4 GEMM of the SVDQuant linear ("Nunchaku Lite", "Supported
// quantization types": svdq_w4a4 nvfp4, group 16; low-rank up-projection and
// bias fused into the epilogue as in the blog "Nunchaku 4-bit inference in
// Diffusers", "Background: SVDQuant and Nunchaku"):
//   y[m,n] = alpha_a*alpha_w * sum_g sa[m,g]*sw[n,g]*P[m,n,g] + XL1.L2 + bias
//
// gfx950's block-scaled matrix instructions scale 32 channels by a power of
// two, while NVFP4 scales 16 channels by an E4M3 number, so the scales are not
// folded into the matrix core.  Instead each operand is dequantized exactly:
// an E2M1 value (at most 2 significant bits) times an E4M3 scale (at most 4)
// has at most 6 significant bits and lies in [2^-10, 2688], so e2m1(c) * s is
// exact in fp16.  Dequantization is two instructions per pair of codes:
// v_cvt_scalef32_pk_f16_fp4 with a unit scale (its scale operand only applies
// a power of two) gives the E2M1 values in fp16, and v_pk_mul_f16 multiplies
// both by the group's scale, exactly.  The tile is expanded to fp16 while
// staging to LDS and the whole K reduction runs on v_mfma_f32_32x32x16_f16
// with fp32 accumulation; there is no per-group rescale on the vector ALUs
// (which would cost more than the matrix work at 16-channel groups).  With
// unit scales the same path yields the exact group products P (multiples of
// 1/4) for the partial-product test mode.
//
// Tiling: 128(n) x 128(m) per 256-thread workgroup, wave tiles of 64x64,
// K steps of 64 channels (four NVFP4 groups) double buffered in LDS.  Codes
// are loaded a pair of steps at a time, four lanes per 64-byte row segment
// (a load instruction with two lanes per 32-byte segment touches twice the
// rows, and those per-lane cache accesses, not bytes, were a third of the
// kernel's time), and scales sixteen steps at a time, 64 bytes per row split
// over a lane quad (a step's scales reach the quad by a DPP broadcast); both
// arrive about two steps before use (branch-free buffer loads, rows past M
// read as zero), and scheduling barriers keep the loads at the top of a step
// and their expansion into LDS at its end (left to itself the compiler moves
// the expansion up to the loads, which makes the step wait for them at
// once).  Tiles are assigned
// so that each XCD works on a contiguous part of a banded order.
#include <type_traits>
#include <utility>

#include "common.h"
#include "launch.h"
#include "mlp_epi.h"
#include "qkv_epi.h"
#include "tail_split.h"

namespace svdq {

typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));

namespace {
constexpr int BM = 128, BN = 128;
constexpr int ROW = 72;  // fp16 per LDS row: 64 channels + 8 padding
constexpr uint32_t kBufDword3 = 0x00020000u;  // raw buffer, 32-bit data format

// f(integral_constant<int, I>) for I = 0, 1, ... in order
template <typename F, int... I>
__device__ __forceinline__ void static_for(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}

// 8 codes of one dword (channels 0..7, even channel in the low nibble) times
// the scale pair s -> 8 fp16 (exact).
__device__ __forceinline__ uint4 dequant8(u32 w, h2 s) {
  const h2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * s;
  const h2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * s;
  const h2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * s;
  const h2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * s;
  return uint4{__builtin_bit_cast(u32, p0), __builtin_bit_cast(u32, p1), __builtin_bit_cast(u32, p2),
               __builtin_bit_cast(u32, p3)};
}
// The two E4M3 scales in the low 16 bits of `bits` -> fp16 (exact: E4M3 values
// are fp16 numbers), each duplicated into a pair.
__device__ __forceinline__ void scale_pairs(u32 bits, h2& s0, h2& s1) {
  const h2 v = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(bits, 1.0f, false);
  s0 = __builtin_shufflevector(v, v, 0, 0);
  s1 = __builtin_shufflevector(v, v, 1, 1);
}
}  // namespace

// MODE 0: Y; 1: fp32 partial products per 16-channel group; 2: Y of the fused
// attention projection (Q/K RMSNorm and rotary embedding in the epilogue);
// 3: the fused MLP up-projection (no Y: GELU, then the down projection's NVFP4
// quantization and low-rank input)
template <int MODE>
__global__ __launch_bounds__(256) void gemm_nvfp4_kernel(
    int M, int N, int K, int rank, const uint8_t* __restrict__ ac, const uint8_t* __restrict__ as,
    float alpha, const uint8_t* __restrict__ wc, const uint8_t* __restrict__ ws,
    const float* __restrict__ xl1, const uint16_t* __restrict__ l2t,
    const uint16_t* __restrict__ bias, uint16_t* __restrict__ y, float* __restrict__ psums, QkvEpi qe,
    MlpEpi me, TailSplit ts) {
  // One array: the activation tiles start 32 bytes past a multiple of 128
  // bytes from the weight tiles, so that a staging store whose lanes write
  // both (the same rows and halves of each) spreads over all the banks.
  __shared__ __align__(16) uint16_t sWX[2 * BN * ROW + 16 + 2 * BM * ROW];
  uint16_t(*const sW)[BN * ROW] = (uint16_t(*)[BN * ROW])sWX;
  uint16_t(*const sX)[BM * ROW] = (uint16_t(*)[BM * ROW])(sWX + 2 * BN * ROW + 16);

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  // XCD-contiguous ranges of a banded tile order (see gemm_int4.hip)
  const int m_tiles = (M + BM - 1) / BM, n_tiles = N / BN;
  const int tiles = m_tiles * n_tiles;
  // the plain GEMM may run its grid's last partial round as K slices
  // (tail_split.h): slices are whole 16-step scale blocks of K
  int t = blockIdx.x, slice = -1, tail_idx = 0;
  if ((tiles & 7) == 0) t = split_tile_of(t, tiles, MODE == 0 || MODE == 2 ? ts : TailSplit{}, slice, tail_idx);
  constexpr int kBandM = 12;
  const int band = t / (kBandM * n_tiles), in_band = t - band * (kBandM * n_tiles);
  const int band_m0 = band * kBandM;
  const int band_h = m_tiles - band_m0 < kBandM ? m_tiles - band_m0 : kBandM;
  const int m0 = (band_m0 + in_band % band_h) * BM, n0 = (in_band / band_h) * BN;
  const int wn = (wave >> 1) * 64, wm = (wave & 1) * 64;
  int steps = K >> 6, st0 = 0;  // this workgroup's steps: [st0, st0 + steps)
  const int G = K >> 4;
  const int rowb = K >> 1;
  if ((MODE == 0 || MODE == 2) && slice >= 0) {
    const int nb = steps >> 4;
    st0 = 16 * (slice * nb / ts.parts);
    steps = 16 * ((slice + 1) * nb / ts.parts) - st0;
  }

  // Staging.  Two K steps (128 channels) are 64 contiguous bytes of codes per
  // row; a load gives each lane 16 of them, four lanes per row, so one load
  // instruction covers 16 whole 64-byte row segments.  Thread t owns rows
  // r0 = t/4 and r0 + 64 of both operands: part p = t%4 of the weight rows
  // and part p^2 of the activation rows.  Parts 0, 1 are the first step of
  // the pair and parts 2, 3 the second, so for either step every thread holds
  // two 32-channel chunks (of the weights for one step, of the activations
  // for the other) and the expansion work is the same on every lane.  The 16
  // E4M3 scale bytes of four steps of a row are one 16-byte load, issued once
  // every four steps.
  const int p = tid & 3, r0 = tid >> 2;
  const __amdgpu_buffer_rsrc_t wres = __builtin_amdgcn_make_buffer_rsrc((void*)wc, (short)0, N * rowb, kBufDword3);
  const __amdgpu_buffer_rsrc_t xres = __builtin_amdgcn_make_buffer_rsrc((void*)ac, (short)0, M * rowb, kBufDword3);
  const __amdgpu_buffer_rsrc_t wsres = __builtin_amdgcn_make_buffer_rsrc((void*)ws, (short)0, MODE != 1 ? N * G : 0, kBufDword3);
  const __amdgpu_buffer_rsrc_t asres = __builtin_amdgcn_make_buffer_rsrc((void*)as, (short)0, MODE != 1 ? M * G : 0, kBufDword3);
  // rows past M read as zero (codes and scales)
  const int wco = (n0 + r0) * rowb + 16 * p + 32 * st0, xco = (m0 + r0) * rowb + 16 * (p ^ 2) + 32 * st0;
  const int wso = (n0 + r0) * G + 4 * st0, xso = (m0 + r0) * G + 4 * st0;

  v16f acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  // Codes of step pair P (steps 2P, 2P+1) go to register set P & 1: pair
  // P + 1 is loaded at the start of step 2P and expanded at the ends of steps
  // 2P + 1 and 2P + 2.  Scales: a row's 64 bytes of sixteen steps (steps
  // 16Q .. 16Q+15) are one segment whose quarter p (steps 16Q+4p .. +3) lane p
  // of each lane quad loads, so a load instruction covers 16 whole 64-byte
  // row segments; a step's dword comes from the quad lane that holds it by a
  // DPP broadcast.  They are loaded at the start of step 16Q - 2 into `nxt`
  // and used from `cur` after the rotation at the end of step 16Q - 1.
  // Loads past the last step use an
  // offset beyond every buffer's range (zeros, no memory access), so every
  // step issues the same loads and the compiler's waits stay exact.
  constexpr int kOffOut = 0x7FFFFFF0;
  uint4 cw[2][2], cx[2][2];  // [set][row r0 + 64 j]
  uint4 cur[2][2], nxt[2][2];  // scale blocks [weight / activation][row r0 + 64 j]
  auto cload = [&](int P, auto setc) {
    constexpr int set = decltype(setc)::value;
    const bool live = 2 * P < steps;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      cw[set][j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(wres, live ? wco + 64 * j * rowb + 64 * P : kOffOut, 0, 0));
      cx[set][j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(xres, live ? xco + 64 * j * rowb + 64 * P : kOffOut, 0, 0));
    }
  };
  auto sload = [&](int Q, uint4 (&blk)[2][2]) {
    if constexpr (MODE != 1) {
      const bool live = 16 * Q < steps;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        blk[0][j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(wsres, live ? wso + 64 * j * G + 64 * Q + 16 * p : kOffOut, 0, 0));
        blk[1][j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(asres, live ? xso + 64 * j * G + 64 * Q + 16 * p : kOffOut, 0, 0));
      }
    } else {
#pragma unroll
      for (int j = 0; j < 2; ++j) blk[0][j] = blk[1][j] = uint4{0x38383838u, 0x38383838u, 0x38383838u, 0x38383838u};  // E4M3 1.0
    }
  };
  // Expand step t into LDS buffer buf: H = t & 1 (step of its pair), CS = its
  // code set, T16 = t & 15 (quad lane T16 / 4 holds its scales, dword T16 % 4).
  auto sstore = [&](int buf, auto Hc, auto CSc, auto T16c, const uint4 (&blk)[2][2]) {
    constexpr int H = decltype(Hc)::value, CS = decltype(CSc)::value, T16 = decltype(T16c)::value;
    constexpr int KD = T16 & 3, QL = T16 >> 2;
    const bool wside = (p < 2) == (H == 0);  // this lane holds weight chunks of step t
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const uint4 c = wside ? cw[CS][j] : cx[CS][j];
      const uint4 bw = blk[0][j], bx = blk[1][j];
      const u32 vw = KD == 0 ? bw.x : KD == 1 ? bw.y : KD == 2 ? bw.z : bw.w;
      const u32 vx = KD == 0 ? bx.x : KD == 1 ? bx.y : KD == 2 ? bx.z : bx.w;
      // quad_perm(QL, QL, QL, QL): every lane of the quad takes lane QL's dword
      const u32 sw4 = (u32)__builtin_amdgcn_mov_dpp((int)vw, QL * 0x55, 0xF, 0xF, true);
      const u32 sx4 = (u32)__builtin_amdgcn_mov_dpp((int)vx, QL * 0x55, 0xF, 0xF, true);
      const u32 sd = wside ? sw4 : sx4;
      h2 s0, s1;
      scale_pairs(sd >> (16 * (p & 1)), s0, s1);  // the chunk's two groups
      uint16_t* dst = (wside ? &sW[buf][0] : &sX[buf][0]) + (r0 + 64 * j) * ROW + 32 * (p & 1);
      *(uint4*)(dst + 0) = dequant8(c.x, s0);
      *(uint4*)(dst + 8) = dequant8(c.y, s0);
      *(uint4*)(dst + 16) = dequant8(c.z, s1);
      *(uint4*)(dst + 24) = dequant8(c.w, s1);
    }
  };

  const int lr = lane & 31, lh = lane >> 5;
  cload(0, std::integral_constant<int, 0>{});
  sload(0, cur);
  sstore(0, std::integral_constant<int, 0>{}, std::integral_constant<int, 0>{}, std::integral_constant<int, 0>{}, cur);
  __syncthreads();

  // step st = 16q + K computes from LDS buffer K & 1 and expands step st + 1
  auto stage = [&](int st, auto Kc) __attribute__((always_inline)) {
    constexpr int K16 = decltype(Kc)::value;
    const int buf = K16 & 1;
    if constexpr ((K16 & 1) == 0) cload((st >> 1) + 1, std::integral_constant<int, ((K16 >> 1) + 1) & 1>{});
    if constexpr (K16 == 14) sload((st >> 4) + 1, nxt);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {  // one NVFP4 group per 16-channel MFMA step
      v8h a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        a[i] = *(const v8h*)&sW[buf][(wn + 32 * i + lr) * ROW + 16 * kk + 8 * lh];
        b[i] = *(const v8h*)&sX[buf][(wm + 32 * i + lr) * ROW + 16 * kk + 8 * lh];
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          if constexpr (MODE == 1) {
            v16f d;
#pragma unroll
            for (int v = 0; v < 16; ++v) d[v] = 0.0f;
            d = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[i], b[j], d, 0, 0, 0);
            const int m = m0 + wm + 32 * j + lr;
            if (m < M) {
#pragma unroll
              for (int v = 0; v < 16; ++v) {
                const int n = n0 + wn + 32 * i + 8 * (v >> 2) + 4 * lh + (v & 3);
                psums[((size_t)m * N + n) * G + 4 * st + kk] = d[v];
              }
            }
          } else {
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[i], b[j], acc[i][j], 0, 0, 0);
          }
        }
    }
    __builtin_amdgcn_sched_barrier(0);
    // past the last step this fills the idle buffer, which nothing reads
    constexpr int T = K16 + 1;
    if constexpr (T < 16)
      sstore(buf ^ 1, std::integral_constant<int, T & 1>{}, std::integral_constant<int, (T >> 1) & 1>{},
             std::integral_constant<int, T>{}, cur);
    else
      sstore(buf ^ 1, std::integral_constant<int, 0>{}, std::integral_constant<int, 0>{},
             std::integral_constant<int, 0>{}, nxt);
    __syncthreads();
  };
  {
    int st = 0;
    for (; st + 15 < steps; st += 16) {
      static_for([&](auto ic) { stage(st + decltype(ic)::value, ic); }, std::make_integer_sequence<int, 16>{});
#pragma unroll
      for (int o = 0; o < 2; ++o)
#pragma unroll
        for (int j = 0; j < 2; ++j) cur[o][j] = nxt[o][j];
    }
    static_for([&](auto ic) { if (st + decltype(ic)::value < steps) stage(st + decltype(ic)::value, ic); },
               std::make_integer_sequence<int, 15>{});
  }

  if constexpr (MODE == 0 || MODE == 2) {
    // a K slice: partials through the workspace; the tile's last slice
    // continues with the sum of all of them (4-float vector k of this lane:
    // acc[k / 8][(k / 4) % 2], elements 4 (k % 4) .. +3)
    if (slice >= 0 &&
        !split_exchange<16>(ts, tail_idx, slice, wave, lane, tid, (unsigned*)sWX,
                            [&](int k) {
                              const v16f& a = acc[k >> 3][(k >> 2) & 1];
                              const int q = 4 * (k & 3);
                              return v4f{a[q], a[q + 1], a[q + 2], a[q + 3]};
                            },
                            [&](int k, v4f v) {
                              v16f& a = acc[k >> 3][(k >> 2) & 1];
                              const int q = 4 * (k & 3);
                              a[q] = v[0];
                              a[q + 1] = v[1];
                              a[q + 2] = v[2];
                              a[q + 3] = v[3];
                            }))
      return;
  }

  if constexpr (MODE != 1) {
    // Inputs of the attention-projection epilogue (MODE 2), issued first so
    // that their latency overlaps the low-rank products: norm weights of this
    // lane's columns and rotary (cos, sin) pairs of its tokens.  The part (Q,
    // K or V) is the same for the whole workgroup (heads * head_dim is a
    // multiple of the 128-column tile).
    const int qpart = MODE == 2 ? qkv_part(n0 + wn, qe) : 2;
    const int qc0 = MODE == 2 ? qkv_channel(n0 + wn, qe) : 0;
    uint2 wv[2][4];
    float4 cs[2][2][4];
    if (MODE == 2 && qpart < 2) {
      const uint16_t* wnorm = qpart == 0 ? qe.norm_q : qe.norm_k;
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) wv[i][q] = *(const uint2*)(wnorm + qc0 + 32 * i + 8 * q + 4 * lh);
      int row[2];
      rope_rows_of<2, 32>(m0 + wm + lr, qe, row);
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int q = 0; q < 4; ++q)
            cs[i][j][q] = qe.rope ? *(const float4*)(qe.rope + (size_t)row[j] * qe.head_dim + qc0 + 32 * i + 8 * q + 4 * lh)
                                  : float4{1.0f, 0.0f, 1.0f, 0.0f};
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] *= alpha;
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
          pk.x = pack_bf16x2(f0.x, f0.y);
          pk.y = pack_bf16x2(f0.z, f0.w);
          pk.z = pack_bf16x2(f1.x, f1.y);
          pk.w = pack_bf16x2(f1.z, f1.w);
        }
        bl[j] = __builtin_bit_cast(v8bf, pk);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al[i], bl[j], acc[i][j], 0, 0, 0);
    }
    if constexpr (MODE == 2) {
      // Fused attention projection (see gemm_int4.hip): bias first, then
      // per-token RMSNorm and rotary embedding of every Q and K head.  This
      // lane holds columns 32i + 8q + 4lh .. +3 of the wave's 64 for tokens
      // 32j + lr.
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int n = n0 + wn + 32 * i + 8 * q + 4 * lh;
          float b[4] = {0.f, 0.f, 0.f, 0.f};
          if (bias) {
            const uint2 bb = *(const uint2*)(bias + n);
            b[0] = bf16_bits_to_f32(bb.x & 0xFFFFu);
            b[1] = bf16_bits_to_f32(bb.x >> 16);
            b[2] = bf16_bits_to_f32(bb.y & 0xFFFFu);
            b[3] = bf16_bits_to_f32(bb.y >> 16);
          }
#pragma unroll
          for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int v = 0; v < 4; ++v) acc[i][j][4 * q + v] += b[v];
        }
      if (qpart < 2) {
        float ss[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          float t = 0.0f;
#pragma unroll
          for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int v = 0; v < 16; ++v) t = fmaf(acc[i][j][v], acc[i][j][v], t);
          ss[j] = sum_over_halves(t);  // the wave's 64 columns
        }
        if (qe.head_dim == 128) {  // the other 64 columns of the head: partner wave (wn ^ 64)
          float* red = (float*)&sW[0][0];  // free after the main loop
          if (lh == 0) {
#pragma unroll
            for (int j = 0; j < 2; ++j) red[wave * 64 + 32 * j + lr] = ss[j];
          }
          __syncthreads();
#pragma unroll
          for (int j = 0; j < 2; ++j) ss[j] += red[(wave ^ 2) * 64 + 32 * j + lr];
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const float r = inv_rms(ss[j], qe);
#pragma unroll
          for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const float4 o = norm_rope4(acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                                          acc[i][j][4 * q + 3], r, wv[i][q], cs[i][j][q]);
              acc[i][j][4 * q] = o.x;
              acc[i][j][4 * q + 1] = o.y;
              acc[i][j][4 * q + 2] = o.z;
              acc[i][j][4 * q + 3] = o.w;
            }
        }
      }
    }
    if constexpr (MODE == 3) {
#pragma clang fp contract(off)
      // Fused MLP up-projection, NVFP4 (the int4 form is in gemm_int4.hip):
      // y + bias -> h = bf16(GELU(y)), then svdq_quantize_act's NVFP4 steps on
      // h: xh = fl32(h * fl32(1/lambda)); per 16-channel group
      // s = e4m3_sat(fl32(amax / fl32(6 alpha))), c = e2m1(fl32(xh * fl32(1 / fl32(s alpha))))
      // (code 0 where s is 0); and XL1 += h . L1 (fp32 atomics: every column
      // tile adds its share).  Y is never written.  This lane holds, for
      // tokens 32j + lr, the columns 32i + 8q + 4lh + v: a 16-channel group
      // (i, q pair) is 8 values here and the other 8 in lane ^ 32.
      const int nw = n0 + wn;
      const int GS = N >> 4;  // scale bytes per row
      const float d6 = 6.0f * me.alpha;
      u32 hp[2][2][4][2];  // [i][j][q]: h as bf16 pairs (v = 0, 1 and 2, 3)
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int n = nw + 32 * i + 8 * q + 4 * lh;
          float b[4] = {0.f, 0.f, 0.f, 0.f};
          if (bias) {
            const uint2 bb = *(const uint2*)(bias + n);
            b[0] = bf16_bits_to_f32(bb.x & 0xFFFFu);
            b[1] = bf16_bits_to_f32(bb.x >> 16);
            b[2] = bf16_bits_to_f32(bb.y & 0xFFFFu);
            b[3] = bf16_bits_to_f32(bb.y >> 16);
          }
          const uint2 lw = me.lam ? *(const uint2*)(me.lam + n) : uint2{0x3F803F80u, 0x3F803F80u};
          const float rl[4] = {1.0f / bf16_bits_to_f32(lw.x & 0xFFFFu), 1.0f / bf16_bits_to_f32(lw.x >> 16),
                               1.0f / bf16_bits_to_f32(lw.y & 0xFFFFu), 1.0f / bf16_bits_to_f32(lw.y >> 16)};
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            float h[4];
#pragma unroll
            for (int v = 0; v < 4; ++v) h[v] = gelu_f32(acc[i][j][4 * q + v] + b[v]);
            hp[i][j][q][0] = pack_bf16x2(h[0], h[1]);
            hp[i][j][q][1] = pack_bf16x2(h[2], h[3]);
            acc[i][j][4 * q] = bf16_bits_to_f32(hp[i][j][q][0] & 0xFFFFu) * rl[0];  // xh
            acc[i][j][4 * q + 1] = bf16_bits_to_f32(hp[i][j][q][0] >> 16) * rl[1];
            acc[i][j][4 * q + 2] = bf16_bits_to_f32(hp[i][j][q][1] & 0xFFFFu) * rl[2];
            acc[i][j][4 * q + 3] = bf16_bits_to_f32(hp[i][j][q][1] >> 16) * rl[3];
          }
        }
      // codes through LDS (free after the main loop): this wave's 64 tokens x
      // 32 bytes; scales: the wave's four group bytes of a token in one dword
      constexpr int CROW = 48;  // bytes per LDS row (32 + pad)
      uint8_t* ct = (uint8_t*)&sW[0][0] + wave * 64 * CROW;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        u32 sb4 = 0u;
#pragma unroll
        for (int g = 0; g < 4; ++g) {  // group g: columns 16g .. 16g+15 of the wave's 64
          const int i = g >> 1, q0 = 2 * (g & 1);
          float xv[8];
          float a = 0.0f;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            xv[e] = acc[i][j][4 * q0 + e];
            a = fmaxf(a, fabsf(xv[e]));
          }
          u32 ab = __float_as_uint(a);
          auto pr = __builtin_amdgcn_permlane32_swap(ab, ab, false, false);  // the partner lane's 8
          a = fmaxf(__uint_as_float(pr[0]), __uint_as_float(pr[1]));
          const u32 sbits = f32_to_e4m3_sat_pos(a / d6);
          const float sf = e4m3_to_f32(sbits);
          float t = 0.0f;
          if (sf != 0.0f) {
            const float sa = sf * me.alpha;
            t = 1.0f / sa;
          }
          // a zero scale writes code 0 (t = 0 would give -0 codes for negative xh)
          const u32 w = sf == 0.0f ? 0u : e2m1_codes8(xv, t);
          // bytes: columns 16g + 4lh + 0..3 (w's low half), 16g + 8 + 4lh + 0..3 (high half)
          *(uint16_t*)(ct + (32 * j + lr) * CROW + 8 * g + 2 * lh) = (uint16_t)(w & 0xFFFFu);
          *(uint16_t*)(ct + (32 * j + lr) * CROW + 8 * g + 4 + 2 * lh) = (uint16_t)(w >> 16);
          sb4 |= sbits << (8 * g);
        }
        const int m = m0 + wm + 32 * j + lr;
        if (lh == 0 && m < M) *(u32*)((uint8_t*)me.scales + (size_t)m * GS + (nw >> 4)) = sb4;
      }
#pragma unroll
      for (int rr = 0; rr < 2; ++rr) {  // 64 rows x 2 halves, 64 lanes per pass
        const int row = rr * 32 + (lane >> 1), half = lane & 1;
        const uint4 v = *(const uint4*)(ct + row * CROW + 16 * half);
        const int m = m0 + wm + row;
        if (m < M) *(uint4*)(me.codes + (size_t)m * (N >> 1) + (nw >> 1) + 16 * half) = v;
      }
      // XL1 += h . L1 on v_mfma_f32_32x32x16_bf16: A = h [32 tokens x 16
      // channels], chunk (i, qp) = columns 32i + 16qp + 0..15 with this lane's
      // own values in its k slots 8lh + 4q' + v (column 32i + 16qp + 8q' + 4lh + v);
      // B = L1 in the same channel order, 32 ranks per block; D lane (rank lr,
      // lh) holds tokens 8(v/4) + 4lh + v%4 of the 32.  The two column waves of
      // a row block (wave and wave ^ 2) cover the same tokens: the second puts
      // its partial in LDS, the first adds it (a fixed order) and makes the
      // one atomic add per element.
      float* const xx = (float*)((uint8_t*)&sW[0][0] + 4 * 64 * CROW);  // [2 row blocks][2 j][16][64]
      const int cw = wave >> 1, rw = wave & 1;
      for (int rb = 0; rb < me.rank; rb += 32) {
        const int r = rb + lr;
        v8bf bl[2][2];
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int qp = 0; qp < 2; ++qp) {
            uint2 lo = {0u, 0u}, hi = {0u, 0u};
            if (r < me.rank) {
              lo = *(const uint2*)(me.l1t + (size_t)r * N + nw + 32 * i + 16 * qp + 4 * lh);
              hi = *(const uint2*)(me.l1t + (size_t)r * N + nw + 32 * i + 16 * qp + 8 + 4 * lh);
            }
            bl[i][qp] = __builtin_bit_cast(v8bf, uint4{lo.x, lo.y, hi.x, hi.y});
          }
        v16f d[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
#pragma unroll
          for (int v = 0; v < 16; ++v) d[j][v] = 0.0f;
#pragma unroll
          for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int qp = 0; qp < 2; ++qp) {
              const v8bf al = __builtin_bit_cast(v8bf, uint4{hp[i][j][2 * qp][0], hp[i][j][2 * qp][1],
                                                             hp[i][j][2 * qp + 1][0], hp[i][j][2 * qp + 1][1]});
              d[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, bl[i][qp], d[j], 0, 0, 0);
            }
        }
        __syncthreads();  // the previous block's readers are done with xx
        if (cw == 1) {
#pragma unroll
          for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) xx[((rw * 2 + j) * 16 + v) * 64 + lane] = d[j][v];
        }
        __syncthreads();
        if (cw == 0 && r < me.rank) {
#pragma unroll
          for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
              const int m = m0 + wm + 32 * j + 8 * (v >> 2) + 4 * lh + (v & 3);
              if (m < M) unsafeAtomicAdd(me.xl1 + (size_t)m * me.rank + r, d[j][v] + xx[((rw * 2 + j) * 16 + v) * 64 + lane]);
            }
        }
      }
      return;
    }
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
          if (MODE == 0 && bias) {
            const uint2 bb = *(const uint2*)(bias + n);
            bv[0] = bf16_bits_to_f32(bb.x & 0xFFFFu);
            bv[1] = bf16_bits_to_f32(bb.x >> 16);
            bv[2] = bf16_bits_to_f32(bb.y & 0xFFFFu);
            bv[3] = bf16_bits_to_f32(bb.y >> 16);
          }
          uint2 o;
          o.x = pack_bf16x2(acc[i][j][4 * q] + bv[0], acc[i][j][4 * q + 1] + bv[1]);
          o.y = pack_bf16x2(acc[i][j][4 * q + 2] + bv[2], acc[i][j][4 * q + 3] + bv[3]);
          *(uint2*)(y + (size_t)m * N + n) = o;
        }
      }
  }
}

// The plain grid's last partial round as K slices of whole 16-step scale
// blocks, with a workspace: the same grids as the int4 GEMM's split (more
// than one round of two tiles per CU, a last round of at most an eighth of a
// round), K of at least two blocks; as many slices as blocks, at most
// kTailParts (the 3072-channel QKV projection: three).
static TailSplit nvfp4_tail_split(int blocks, int steps, void* work) {
  TailSplit ts{};
  const int slots = 2 * device_cu_count(), nb = steps / 16;
  if (!work || (blocks & 7) || (slots & 7) || blocks <= slots || (steps % 16) || nb < 2) return ts;
  const int tail = blocks % slots;
  if (tail == 0 || tail > slots / 8 || tail > kTailMaxTiles) return ts;
  ts.full = blocks - tail;
  ts.tail = tail;
  ts.parts = nb < kTailParts ? nb : kTailParts;
  ts.part = (float*)work;
  ts.cnt = (unsigned*)((uint8_t*)work + kTailPartBytes);
  return ts;
}

hipError_t launch_gemm_nvfp4(const GemmArgs& a, hipStream_t st) {
  const int m_tiles = (int)((a.M + BM - 1) / BM);
  const int blocks = m_tiles * (int)(a.N / BN);  // N % 128 == 0
  const QkvEpi none{};
  const MlpEpi mnone{};
  const TailSplit tnone{};
  if (a.psums) {
    hipLaunchKernelGGL(gemm_nvfp4_kernel<1>, dim3(blocks), dim3(256), 0, st, (int)a.M, (int)a.N,
                       (int)a.K, 0, (const uint8_t*)a.act_codes, nullptr, 1.0f,
                       (const uint8_t*)a.w_codes, nullptr, nullptr, nullptr, nullptr, nullptr,
                       (float*)a.psums, none, mnone, tnone);
  } else if (a.qkv) {
    const TailSplit ts = nvfp4_tail_split(blocks, (int)(a.K / 64), a.work);
    const int grid = ts.parts > 0 ? ts.full + ts.tail * ts.parts : blocks;
    hipLaunchKernelGGL(gemm_nvfp4_kernel<2>, dim3(grid), dim3(256), 0, st, (int)a.M, (int)a.N,
                       (int)a.K, a.rank, (const uint8_t*)a.act_codes, (const uint8_t*)a.act_scales,
                       a.alpha_a * a.alpha_w, (const uint8_t*)a.w_codes, (const uint8_t*)a.w_scales,
                       a.xl1, (const uint16_t*)a.l2t, (const uint16_t*)a.bias, (uint16_t*)a.y, nullptr,
                       *a.qkv, mnone, ts);
  } else if (a.mlp) {
    const int nx = (int)(a.M * a.mlp->rank);
    if (nx > 0) hipLaunchKernelGGL(fill_zero_f32, dim3((nx + 255) / 256), dim3(256), 0, st, a.mlp->xl1, nx);
    hipLaunchKernelGGL(gemm_nvfp4_kernel<3>, dim3(blocks), dim3(256), 0, st, (int)a.M, (int)a.N,
                       (int)a.K, a.rank, (const uint8_t*)a.act_codes, (const uint8_t*)a.act_scales,
                       a.alpha_a * a.alpha_w, (const uint8_t*)a.w_codes, (const uint8_t*)a.w_scales,
                       a.xl1, (const uint16_t*)a.l2t, (const uint16_t*)a.bias, nullptr, nullptr, none, *a.mlp,
                       tnone);
  } else {
    const TailSplit ts = nvfp4_tail_split(blocks, (int)(a.K / 64), a.work);
    const int grid = ts.parts > 0 ? ts.full + ts.tail * ts.parts : blocks;
    hipLaunchKernelGGL(gemm_nvfp4_kernel<0>, dim3(grid), dim3(256), 0, st, (int)a.M, (int)a.N,
                       (int)a.K, a.rank, (const uint8_t*)a.act_codes, (const uint8_t*)a.act_scales,
                       a.alpha_a * a.alpha_w, (const uint8_t*)a.w_codes, (const uint8_t*)a.w_scales,
                       a.xl1, (const uint16_t*)a.l2t, (const uint16_t*)a.bias, (uint16_t*)a.y, nullptr, none,
                       mnone, ts);
  }
  return hipGetLastError();
}

}  // namespace svdq
