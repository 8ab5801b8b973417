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
        const u32 sbits = f32_to_f16_sat_bits(amax / 7.0f);
        const float sf = f16_bits_to_f32(sbits);
        const float t = sf == 0.0f ? 0.0f : 1.0f / sf;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          float q = __builtin_rintf(xh[i] * t);
          q = fminf(fmaxf(q, -8.0f), 7.0f);
          const u32 nib = (u32)(int)q & 0xFu;
          if (i < 8) pk0 |= nib << (4 * i);
          else pk1 |= nib << (4 * (i - 8));
        }
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
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const u32 nib = sf == 0.0f ? 0u : f32_to_e2m1_sat(xh[i] * t);
          if (i < 8) pk0 |= nib << (4 * i);
          else pk1 |= nib << (4 * (i - 8));
        }
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

template <int PREC, int RB>
static hipError_t launch_quant(const QuantArgs& a, hipStream_t st) {
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
