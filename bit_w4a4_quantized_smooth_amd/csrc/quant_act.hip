// Activation quantizer of the SVDQuant W4A4 linear, with the low-rank
// down-projection fused in so X is read from HBM exactly once (blog "Nunchaku
// 4-bit inference in Diffusers", "Background: SVDQuant and Nunchaku": the
// down-projection of the 16-bit branch is fused with the quantization kernel).
// Precisions and group sizes from "Nunchaku Lite", "Supported quantization
// types": int4 / group 64 and nvfp4 / group 16.
//
// Work split: one workgroup (8 wave64) owns 16 rows of X and all K.  Wave w
// takes the 64-channel steps s = w, w+8, ..., keeping a few of them in flight
// in a ring of register slots (X and the L1^T slices, as branch-free buffer
// loads; rows past M read as zero).  Within a step lane l holds row
// l % 16 and channels 16*(l/16) .. +16 (two 16-byte loads, 512 contiguous
// bytes per row per workgroup step).  That is also the operand layout of
// v_mfma_f32_16x16x32_bf16, so the raw bf16 X registers feed the matrix core
// for X.L1 directly; the waves' partial XL1 tiles are summed in LDS in a
// fixed order (deterministic).
//
// Numerics: every quantization decision is taken in fp32 with the operations
// written out one by one (no contraction), so codes and scales are bit-exact
// functions of the inputs:
//   xh = fl32(x * fl32(1/lambda))          reciprocal table in LDS, IEEE division
//   int4:  s = fp16_sat(fl32(amax / 7)),  q = clamp(rne(fl32(xh * fl32(1/s))), -8, 7)
//   nvfp4: s = e4m3_sat(fl32(amax / fl32(6*alpha))),
//          c = e2m1_sat(fl32(xh * fl32(1 / fl32(s*alpha))))
#pragma clang fp contract(off)

#include "common.h"
#include "launch.h"

namespace svdq {

// Eight waves per workgroup; with at most 128 VGPRs (ranks up to 32) two
// workgroups share a CU, so a DiT-sized call (a few hundred workgroups) is
// resident at once.  Each wave keeps W of its 64-channel steps in flight in a
// ring of register slots (a step also carries RB*2 fragments of L1^T, so W
// shrinks as the rank grows): step j is computed while steps j+1 .. j+W-1
// are loading, and its slot is refilled with step j+W right after.
template <int RB>
struct QuantCfg {
  static constexpr int WAVES = 8;
  static constexpr int NT = WAVES * 64;
  static constexpr int W = RB <= 1 ? 3 : RB <= 4 ? 2 : 1;
};

// Max over lanes l, l^16, l^32 and l^48: the four 16-channel slices of one
// row's 64-channel group.  The permlane swaps move whole 16-lane rows without
// going through LDS.
__device__ __forceinline__ float max_over_rows(float v) {
  u32 bv = __float_as_uint(v);
  auto p = __builtin_amdgcn_permlane16_swap(bv, bv, false, false);
  v = fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
  bv = __float_as_uint(v);
  auto q = __builtin_amdgcn_permlane32_swap(bv, bv, false, false);
  return fmaxf(__uint_as_float(q[0]), __uint_as_float(q[1]));
}

template <int PREC, int RB>
__global__ __launch_bounds__(QuantCfg<RB>::NT) void quant_act_kernel(
    int M, int K, const uint16_t* __restrict__ x, const uint16_t* __restrict__ lam,
    const uint16_t* __restrict__ l1t, float alpha, uint8_t* __restrict__ codes,
    void* __restrict__ scales, float* __restrict__ xl1) {
  constexpr int WAVES = QuantCfg<RB>::WAVES, NT = QuantCfg<RB>::NT, W = QuantCfg<RB>::W;
  constexpr int RBX = RB > 0 ? RB : 1;
  constexpr int kOut = 0x7FFFFFF0;  // offset past num_records: the load returns 0
  extern __shared__ __align__(16) float smem[];
  float* rl = smem;   // [K] fp32 reciprocals of lambda (main loop)
  float* red = smem;  // [WAVES][16 rows][RB*16] partial XL1 (after it, same space)
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int row0 = blockIdx.x * 16;
  const int r = lane & 15, c = lane >> 4;
  const int m = row0 + r;
  const bool valid = m < M;
  const int nsteps = K >> 6;
  // this wave's steps are wave + WAVES * j, j < nst
  const int nst = nsteps > wave ? (nsteps - wave + WAVES - 1) / WAVES : 0;

  // Raw buffer loads with every offset in the range-checked vector operand:
  // rows past M and steps past the end read zeros, with no branches.
  const __amdgpu_buffer_rsrc_t xres = __builtin_amdgcn_make_buffer_rsrc((void*)x, (short)0, M * K * 2, 0x00020000);
  const __amdgpu_buffer_rsrc_t lres = __builtin_amdgcn_make_buffer_rsrc((void*)l1t, (short)0, RB * 16 * K * 2, 0x00020000);
  const u32 xo = (u32)m * (u32)K * 2u + 32u * c;  // step 0, first 16 bytes of this lane
  u32 lo[RBX];
#pragma unroll
  for (int rb = 0; rb < RBX; ++rb) lo[rb] = (u32)(rb * 16 + r) * (u32)K * 2u + 32u * c;

  uint4 xa[W], xb[W];
  uint4 lb[W][RBX][2];
  auto issue = [&](int u, int j) {  // load step j of this wave into slot u
    const int st = wave + WAVES * j;
    const bool live = j < nst;
    const u32 sb = 128u * st;
    xa[u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(xres, live ? xo + sb : kOut, 0, 0));
    xb[u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(xres, live ? xo + sb + 16 : kOut, 0, 0));
    if constexpr (RB > 0) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        lb[u][rb][0] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(lres, live ? lo[rb] + sb : kOut, 0, 0));
        lb[u][rb][1] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(lres, live ? lo[rb] + sb + 16 : kOut, 0, 0));
      }
    }
  };
  // the first W steps are in flight before the reciprocal table is built
#pragma unroll
  for (int u = 0; u < W; ++u) issue(u, u);

  // lambda reciprocals: 8 channels per 16-byte load, every load of this
  // thread issued before the first division (K <= 32768: at most 8 each)
  {
    const __amdgpu_buffer_rsrc_t lamres = __builtin_amdgcn_make_buffer_rsrc((void*)lam, (short)0, lam ? K * 2 : 0, 0x00020000);
    constexpr int LCH = 8;
    uint4 lv[LCH];
#pragma unroll
    for (int i = 0; i < LCH; ++i) {
      const int ch = tid + NT * i;  // 8-channel chunk
      lv[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(lamres, ch * 8 < K ? ch * 16 : kOut, 0, 0));
    }
#pragma unroll
    for (int i = 0; i < LCH; ++i) {
      const int ch = tid + NT * i;
      if (ch * 8 >= K) break;
      const u32 w4[4] = {lv[i].x, lv[i].y, lv[i].z, lv[i].w};
      float o[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        o[2 * e] = lam ? 1.0f / bf16_bits_to_f32(w4[e] & 0xFFFFu) : 1.0f;
        o[2 * e + 1] = lam ? 1.0f / bf16_bits_to_f32(w4[e] >> 16) : 1.0f;
      }
      *(float4*)&rl[ch * 8] = float4{o[0], o[1], o[2], o[3]};
      *(float4*)&rl[ch * 8 + 4] = float4{o[4], o[5], o[6], o[7]};
    }
  }
  __syncthreads();

  v4f acc[RBX];
#pragma unroll
  for (int i = 0; i < RBX; ++i) acc[i] = v4f{0.f, 0.f, 0.f, 0.f};
  const float d6 = 6.0f * alpha;

  for (int j0 = 0; j0 < nst; j0 += W) {
#pragma unroll
    for (int u = 0; u < W; ++u) {
      const int j = j0 + u;
      if (j >= nst) break;  // wave-uniform
      const int st = wave + WAVES * j;
      const int k0 = (st << 6) + (c << 4);
      const uint4 va = xa[u], vb = xb[u];
      const u32 xw[8] = {va.x, va.y, va.z, va.w, vb.x, vb.y, vb.z, vb.w};
      float rk[16];
      *(float4*)&rk[0] = *(const float4*)&rl[k0];
      *(float4*)&rk[4] = *(const float4*)&rl[k0 + 4];
      *(float4*)&rk[8] = *(const float4*)&rl[k0 + 8];
      *(float4*)&rk[12] = *(const float4*)&rl[k0 + 12];
      float xh[16];
      float amax = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        xh[2 * i] = bf16_bits_to_f32(xw[i] & 0xFFFFu) * rk[2 * i];
        xh[2 * i + 1] = bf16_bits_to_f32(xw[i] >> 16) * rk[2 * i + 1];
        amax = fmaxf(amax, fmaxf(fabsf(xh[2 * i]), fabsf(xh[2 * i + 1])));
      }

      u32 pk0 = 0u, pk1 = 0u;
      if constexpr (PREC == 0) {
        amax = max_over_rows(amax);  // one 64-channel group = lanes l, l^16, l^32, l^48
        const u32 sbits = f32_to_f16_sat_bits(div7_rn(amax));
        const float sf = f16_bits_to_f32(sbits);
        const float t = sf == 0.0f ? 0.0f : 1.0f / sf;
        pk0 = int4_codes8(xh, t);
        pk1 = int4_codes8(xh + 8, t);
        if (valid) {
          *(uint2*)(codes + (size_t)m * (K >> 1) + (k0 >> 1)) = uint2{pk0, pk1};
          if (c == 0) ((uint16_t*)scales)[(size_t)m * (K >> 6) + st] = (uint16_t)sbits;
        }
      } else {
        // one 16-channel group = this lane's 16 channels
        const u32 sbits = f32_to_e4m3_sat_pos(amax / d6);
        const float sf = e4m3_to_f32(sbits);
        float t = 0.0f;
        if (sf != 0.0f) {
          const float sa = sf * alpha;
          t = 1.0f / sa;
        }
        // a zero scale writes code 0 (t = 0 would give -0 codes for negative xh)
        pk0 = sf == 0.0f ? 0u : e2m1_codes8(xh, t);
        pk1 = sf == 0.0f ? 0u : e2m1_codes8(xh + 8, t);
        if (valid) {
          *(uint2*)(codes + (size_t)m * (K >> 1) + (k0 >> 1)) = uint2{pk0, pk1};
          ((uint8_t*)scales)[(size_t)m * (K >> 4) + (st << 2) + c] = (uint8_t)sbits;
        }
      }

      if constexpr (RB > 0) {
        // XL1 += X[16 rows, these 64 channels] . L1[these channels, 16*RB]
        const v8bf a0 = __builtin_bit_cast(v8bf, va);
        const v8bf a1 = __builtin_bit_cast(v8bf, vb);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          acc[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, __builtin_bit_cast(v8bf, lb[u][rb][0]), acc[rb], 0, 0, 0);
          acc[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, __builtin_bit_cast(v8bf, lb[u][rb][1]), acc[rb], 0, 0, 0);
        }
      }
      issue(u, j + W);  // refill this slot (past the end: zeros, never used)
    }
  }

  if constexpr (RB > 0) {
    constexpr int R = RB * 16;
    // lane holds D[row 4*(lane/16) + v][col lane%16] of each 16x16 block;
    // the partial tiles overwrite the reciprocal table once every wave is done
    __syncthreads();
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int v = 0; v < 4; ++v) red[(wave * 16 + 4 * c + v) * R + rb * 16 + r] = acc[rb][v];
    __syncthreads();
    for (int idx = tid; idx < 16 * R; idx += NT) {
      const int rr = idx / R, col = idx - rr * R;
      float sum = red[rr * R + col];
#pragma unroll
      for (int w = 1; w < WAVES; ++w) sum += red[(w * 16 + rr) * R + col];  // fixed order
      if (row0 + rr < M) xl1[(size_t)(row0 + rr) * R + col] = sum;
    }
  }
}

// Second kernel, for ranks 16 and 32 on calls with more 16-row blocks than
// the device has CUs: the step operands travel through LDS.  Both operands
// of X.L1 are row-major with rows K*2 bytes apart, so loading them straight
// in the matrix-core lane layout (lane = row l%16, as the kernel above does)
// makes every lane of a load touch a different row: one cache access per
// lane, and the address units saturate.  Here X and L1^T slices are copied
// global -> LDS with buffer_load ... lds, lanes 8i .. 8i+7 reading one
// 128-byte row segment (whole-line accesses, no registers), and the lanes
// then read their fragments from LDS.  Codes and scales are the same
// function of the inputs as above (the same fp32 steps); XL1 sums its fp32
// partial products in another fixed order.
//
// Workgroup = 32 rows of X (two 16-row blocks) x 8 waves: wave w takes row
// block w/4 and the steps w%4, w%4 + 4, ... of each chunk, so the two waves
// of a step lane work on the same steps and share one L1^T slice.  A ring of
// three LDS slots per wave (X) and per step lane (L1^T) keeps two steps in
// flight; one barrier per step publishes a slot and frees the oldest.  In LDS
// the 16-byte pieces of a 128-byte row segment are stored XOR-swizzled by the
// row (piece p of row i at slot p ^ (i & 7)), so the fragment reads of 16
// rows spread over the banks.
namespace dma {
constexpr int KC = 2048;  // channels per chunk: 32 steps, 8 per step lane
constexpr int NT = 512;
typedef __attribute__((address_space(3))) void lds_void;

// s_waitcnt with vmcnt = n (0..63), lgkmcnt = 0, expcnt untouched
#define SVDQ_WAIT_VM_LGKM0(n) __builtin_amdgcn_s_waitcnt(((n) & 0xF) | (((n) >> 4) << 14) | 0x0070)

__device__ __forceinline__ int swz(int row, int piece) { return (piece ^ (row & 7)) << 4; }

// 16 bytes per lane, global (buffer offset off) -> LDS at dst + 16 * lane
__device__ __forceinline__ void copy16(__amdgpu_buffer_rsrc_t res, uint8_t* dst, int off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(res, (lds_void*)dst, 16, off, 0, 0, 0);
}
}  // namespace dma

template <int PREC, int RB>
__global__ __launch_bounds__(dma::NT) void quant_act_dma_kernel(
    int M, int K, const uint16_t* __restrict__ x, const uint16_t* __restrict__ lam,
    const uint16_t* __restrict__ l1t, float alpha, uint8_t* __restrict__ codes,
    void* __restrict__ scales, float* __restrict__ xl1) {
  using namespace dma;
  static_assert(RB <= 2, "LDS holds L1^T slices of at most 32 ranks");
  constexpr int RBX = RB > 0 ? RB : 1;
  constexpr int LSL = RBX * 2048;   // bytes of one step's L1^T slice (16*RB rows x 128 B)
  constexpr int NDMA = 2 + RB;      // copies per wave per step: 2 for X, RB for L1^T (8 rows each)
  constexpr int kOut = 0x7FFFFFF0;  // offset past num_records: zeros, no memory access
  constexpr int CROW = KC / 2 + 16; // bytes per codes row in LDS
  __shared__ __align__(16) float rl[KC];                    // lambda reciprocals of the chunk
  __shared__ __align__(16) uint8_t ctile[32][CROW];         // codes of the chunk (XL1 partials at the end)
  __shared__ __align__(16) uint8_t stile[32][KC / 16];      // scales of the chunk
  __shared__ __align__(16) uint8_t xs0[8][2048], xs1[8][2048], xs2[8][2048];  // X slices per wave
  __shared__ __align__(16) uint8_t ls0[4][LSL], ls1[4][LSL], ls2[4][LSL];     // L1^T slices per step lane

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rbk = wave >> 2, sl = wave & 3;  // row block, step lane
  const int row0 = blockIdx.x * 32;
  const int r = lane & 15, c = lane >> 4;

  const __amdgpu_buffer_rsrc_t xres = __builtin_amdgcn_make_buffer_rsrc((void*)x, (short)0, M * K * 2, 0x00020000);
  const __amdgpu_buffer_rsrc_t lres = __builtin_amdgcn_make_buffer_rsrc((void*)l1t, (short)0, RB * 16 * K * 2, 0x00020000);
  const __amdgpu_buffer_rsrc_t lamres = __builtin_amdgcn_make_buffer_rsrc((void*)lam, (short)0, lam ? K * 2 : 0, 0x00020000);
  // copy lanes: lane l moves piece (l%8) ^ swizzle of row l/8 of an 8-row group
  const int cr = lane >> 3;
  u32 xdo[2], ldo[RBX];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int ri = 8 * i + cr;  // row within the 16-row X slice
    xdo[i] = (u32)(row0 + 16 * rbk + ri) * (u32)K * 2u + (u32)(((lane & 7) ^ (ri & 7)) << 4);
  }
#pragma unroll
  for (int i = 0; i < RBX; ++i) {
    const int ri = 8 * (RB * rbk + i) + cr;  // L1^T row: this wave copies rows 8*RB*rbk .. +8*RB
    ldo[i] = (u32)ri * (u32)K * 2u + (u32)(((lane & 7) ^ (ri & 7)) << 4);
  }

  v4f acc[RBX];
#pragma unroll
  for (int i = 0; i < RBX; ++i) acc[i] = v4f{0.f, 0.f, 0.f, 0.f};
  const float d6 = 6.0f * alpha;

  for (int c0 = 0; c0 < K; c0 += KC) {
    const int kc = K - c0 < KC ? K - c0 : KC;
    const int nsteps = kc >> 6;
    const int nst = nsteps > sl ? (nsteps - sl + 3) >> 2 : 0;  // this step lane's steps
    const int J = (nsteps + 3) >> 2;                           // rounds (the step lane 0 count)

    // copy local step j of this wave into slot buffers (xb, lb); past the end:
    // out-of-range offsets (zeros, no memory access), so every wave issues the
    // same number of copies in every round and the waits count exactly
    auto issue = [&](int j, uint8_t(*xb)[2048], uint8_t(*lb)[LSL]) __attribute__((always_inline)) {
      const bool live = j < nst;
      const u32 sb = 128u * (u32)((c0 >> 6) + sl + 4 * j);
#pragma unroll
      for (int i = 0; i < 2; ++i)
        copy16(xres, xb[wave] + 1024 * i, live ? (int)(xdo[i] + sb) : kOut);
      if constexpr (RB > 0) {
#pragma unroll
        for (int i = 0; i < RB; ++i)
          copy16(lres, lb[sl] + 1024 * (RB * rbk + i), live ? (int)(ldo[i] + sb) : kOut);
      }
    };

    // quantize local step j from slot buffers (xb, lb) and add its X.L1 share
    auto compute = [&](int j, uint8_t(*xb)[2048], uint8_t(*lb)[LSL]) __attribute__((always_inline)) {
      const int ls = sl + 4 * j;             // step within the chunk
      const int k0 = (ls << 6) + (c << 4);   // this lane's first channel within the chunk
      const uint8_t* xrow = xb[wave] + r * 128;
      const uint4 va = *(const uint4*)(xrow + swz(r, 2 * c));
      const uint4 vb = *(const uint4*)(xrow + swz(r, 2 * c + 1));
      const u32 xw[8] = {va.x, va.y, va.z, va.w, vb.x, vb.y, vb.z, vb.w};
      float rk[16];
      *(float4*)&rk[0] = *(const float4*)&rl[k0];
      *(float4*)&rk[4] = *(const float4*)&rl[k0 + 4];
      *(float4*)&rk[8] = *(const float4*)&rl[k0 + 8];
      *(float4*)&rk[12] = *(const float4*)&rl[k0 + 12];
      float xh[16];
      float amax = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        xh[2 * i] = bf16_bits_to_f32(xw[i] & 0xFFFFu) * rk[2 * i];
        xh[2 * i + 1] = bf16_bits_to_f32(xw[i] >> 16) * rk[2 * i + 1];
        amax = fmaxf(amax, fmaxf(fabsf(xh[2 * i]), fabsf(xh[2 * i + 1])));
      }
      u32 pk0 = 0u, pk1 = 0u;
      const int trow = 16 * rbk + r;  // row within the workgroup's 32
      if constexpr (PREC == 0) {
        amax = max_over_rows(amax);  // one 64-channel group = lanes l, l^16, l^32, l^48
        const u32 sbits = f32_to_f16_sat_bits(div7_rn(amax));
        const float sf = f16_bits_to_f32(sbits);
        const float t = sf == 0.0f ? 0.0f : 1.0f / sf;
        pk0 = int4_codes8(xh, t);
        pk1 = int4_codes8(xh + 8, t);
        if (c == 0) *(uint16_t*)(&stile[trow][2 * ls]) = (uint16_t)sbits;
      } else {
        // one 16-channel group = this lane's 16 channels
        const u32 sbits = f32_to_e4m3_sat_pos(amax / d6);
        const float sf = e4m3_to_f32(sbits);
        float t = 0.0f;
        if (sf != 0.0f) {
          const float sa = sf * alpha;
          t = 1.0f / sa;
        }
        // a zero scale writes code 0 (t = 0 would give -0 codes for negative xh)
        pk0 = sf == 0.0f ? 0u : e2m1_codes8(xh, t);
        pk1 = sf == 0.0f ? 0u : e2m1_codes8(xh + 8, t);
        stile[trow][4 * ls + c] = (uint8_t)sbits;
      }
      *(uint2*)(&ctile[trow][k0 >> 1]) = uint2{pk0, pk1};
      if constexpr (RB > 0) {
        // XL1 += X[16 rows, these 64 channels] . L1[these channels, 16*RB]
        const v8bf a0 = __builtin_bit_cast(v8bf, va);
        const v8bf a1 = __builtin_bit_cast(v8bf, vb);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          const int lr = rb * 16 + r;  // L1^T row = rank
          const uint8_t* lrow = lb[sl] + lr * 128;
          const uint4 b0 = *(const uint4*)(lrow + swz(lr, 2 * c));
          const uint4 b1 = *(const uint4*)(lrow + swz(lr, 2 * c + 1));
          acc[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, __builtin_bit_cast(v8bf, b0), acc[rb], 0, 0, 0);
          acc[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, __builtin_bit_cast(v8bf, b1), acc[rb], 0, 0, 0);
        }
      }
    };

    // the first two steps in flight while the reciprocal table is built
    issue(0, xs0, ls0);
    issue(1, xs1, ls1);
    if (tid * 8 < kc) {
      const uint4 lv = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(lamres, (c0 + tid * 8) * 2, 0, 0));
      const u32 w4[4] = {lv.x, lv.y, lv.z, lv.w};
      float o[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        o[2 * e] = lam ? 1.0f / bf16_bits_to_f32(w4[e] & 0xFFFFu) : 1.0f;
        o[2 * e + 1] = lam ? 1.0f / bf16_bits_to_f32(w4[e] >> 16) : 1.0f;
      }
      *(float4*)&rl[tid * 8] = float4{o[0], o[1], o[2], o[3]};
      *(float4*)&rl[tid * 8 + 4] = float4{o[4], o[5], o[6], o[7]};
    }

    // Round j: wait for this wave's copies of step j (the NDMA copies of
    // step j+1 may stay in flight) and its LDS reads, barrier (every wave's
    // copies of step j have landed; every wave is done with the slot of step
    // j-1), refill that slot with step j+2, compute step j.
    auto round = [&](int j, uint8_t(*xa)[2048], uint8_t(*la)[LSL], uint8_t(*xc)[2048], uint8_t(*lc)[LSL])
        __attribute__((always_inline)) {
      SVDQ_WAIT_VM_LGKM0(NDMA);
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      issue(j + 2, xc, lc);
      if (j < nst) compute(j, xa, la);  // wave-uniform
    };
    int j = 0;
    for (; j + 3 <= J; j += 3) {
      round(j, xs0, ls0, xs2, ls2);
      round(j + 1, xs1, ls1, xs0, ls0);
      round(j + 2, xs2, ls2, xs1, ls1);
    }
    if (j < J) round(j, xs0, ls0, xs2, ls2);
    if (j + 1 < J) round(j + 1, xs1, ls1, xs0, ls0);
    __syncthreads();  // every copy and every code and scale of the chunk in LDS

    // the chunk's codes and scales out: LDS reads first, then the stores
    {
      const int cpr = kc >> 5;  // 16-byte code pieces per row
      constexpr int CIT = 32 * (KC / 32) / NT;
      uint4 cv[CIT];
      int cdst[CIT];
#pragma unroll
      for (int i = 0; i < CIT; ++i) {
        const int idx = tid + NT * i;
        const int rr = idx / cpr, off = (idx - rr * cpr) << 4;
        const bool ok = idx < 32 * cpr && row0 + rr < M;
        cv[i] = ok ? *(const uint4*)(&ctile[rr][off]) : uint4{0u, 0u, 0u, 0u};
        cdst[i] = ok ? (row0 + rr) * (K >> 1) + (c0 >> 1) + off : -1;
      }
      const int sb = PREC == 0 ? 2 * (kc >> 6) : (kc >> 4);   // scale bytes of the chunk per row (even)
      const int sbr = PREC == 0 ? 2 * (K >> 6) : (K >> 4);    // scale bytes per row
      const int s0b = PREC == 0 ? 2 * (c0 >> 6) : (c0 >> 4);  // first scale byte of the chunk
      constexpr int SIT = 32 * ((PREC == 0 ? 2 * (KC >> 6) : (KC >> 4)) / 2) / NT;
      uint16_t sv[SIT];
      int sdst[SIT];
#pragma unroll
      for (int i = 0; i < SIT; ++i) {
        const int idx = tid + NT * i;
        const int rr = idx / (sb >> 1), off = (idx - rr * (sb >> 1)) << 1;
        const bool ok = idx < 32 * (sb >> 1) && row0 + rr < M;
        sv[i] = ok ? *(const uint16_t*)(&stile[rr][off]) : (uint16_t)0;
        sdst[i] = ok ? (row0 + rr) * sbr + s0b + off : -1;
      }
#pragma unroll
      for (int i = 0; i < CIT; ++i)
        if (cdst[i] >= 0) *(uint4*)(codes + cdst[i]) = cv[i];
#pragma unroll
      for (int i = 0; i < SIT; ++i)
        if (sdst[i] >= 0) *(uint16_t*)((uint8_t*)scales + sdst[i]) = sv[i];
    }
    __syncthreads();  // rl, ctile, stile and the slots are rewritten by the next chunk
  }

  if constexpr (RB > 0) {
    constexpr int R = RB * 16;
    // per-wave partial XL1 tiles [16 rows][R] in the codes tile (free now),
    // summed over the four step lanes of each row block in a fixed order;
    // lane holds D[row 4*(lane/16) + v][col lane%16] of each 16x16 block
    float* red = (float*)&ctile[0][0];
    static_assert(8 * 16 * R * 4 <= 32 * CROW, "partial XL1 tiles fit in the codes tile");
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int v = 0; v < 4; ++v) red[(wave * 16 + 4 * c + v) * R + rb * 16 + r] = acc[rb][v];
    __syncthreads();
    for (int idx = tid; idx < 32 * R; idx += NT) {
      const int rr = idx / R, col = idx - rr * R;  // row within the 32
      const int b = rr >> 4, ri = rr & 15;
      float sum = red[((4 * b) * 16 + ri) * R + col];
#pragma unroll
      for (int s2 = 1; s2 < 4; ++s2) sum += red[((4 * b + s2) * 16 + ri) * R + col];  // fixed order
      if (row0 + rr < M) xl1[(size_t)(row0 + rr) * R + col] = sum;
    }
  }
}

template <int PREC, int RB>
static hipError_t launch_quant_dma(const QuantArgs& a, hipStream_t st) {
  const int blocks = (int)((a.M + 31) / 32);
  hipLaunchKernelGGL((quant_act_dma_kernel<PREC, RB>), dim3(blocks), dim3(dma::NT), 0, st, (int)a.M, (int)a.K,
                     (const uint16_t*)a.x, (const uint16_t*)a.smooth, (const uint16_t*)a.l1t,
                     a.alpha, (uint8_t*)a.codes, a.scales, a.xl1);
  return hipGetLastError();
}

template <int PREC, int RB>
static hipError_t launch_quant(const QuantArgs& a, hipStream_t st) {
  // Ranks 16 / 32: once the 16-row workgroups of the kernel above no longer
  // fit one per CU, the LDS-staged kernel (32 rows per workgroup, coalesced
  // copies) is faster, for both precisions; below that the one-row-block
  // workgroups keep every CU busy.
  if constexpr (RB == 1 || RB == 2) {
    if ((a.M + 15) / 16 > device_cu_count()) return launch_quant_dma<PREC, RB>(a, st);
  }
  const size_t red = RB > 0 ? (size_t)QuantCfg<RB>::WAVES * 16 * RB * 16 : 0;
  const size_t lds = sizeof(float) * ((size_t)a.K > red ? (size_t)a.K : red);
  auto kern = quant_act_kernel<PREC, RB>;
  if (lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  const int blocks = (int)((a.M + 15) / 16);
  hipLaunchKernelGGL(kern, dim3(blocks), dim3(QuantCfg<RB>::NT), lds, st, (int)a.M, (int)a.K,
                     (const uint16_t*)a.x, (const uint16_t*)a.smooth, (const uint16_t*)a.l1t,
                     a.alpha, (uint8_t*)a.codes, a.scales, a.xl1);
  return hipGetLastError();
}

template <int PREC>
static hipError_t dispatch_rank(const QuantArgs& a, hipStream_t st) {
  switch (a.rank / 16) {
    case 0: return launch_quant<PREC, 0>(a, st);
    case 1: return launch_quant<PREC, 1>(a, st);
    case 2: return launch_quant<PREC, 2>(a, st);
    case 3: return launch_quant<PREC, 3>(a, st);
    case 4: return launch_quant<PREC, 4>(a, st);
    case 5: return launch_quant<PREC, 5>(a, st);
    case 6: return launch_quant<PREC, 6>(a, st);
    case 7: return launch_quant<PREC, 7>(a, st);
    case 8: return launch_quant<PREC, 8>(a, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_quantize_act(const QuantArgs& a, hipStream_t st) {
  return a.precision == 0 ? dispatch_rank<0>(a, st) : dispatch_rank<1>(a, st);
}

}  // namespace svdq
