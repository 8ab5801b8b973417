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

#include <type_traits>

#include "awq_small.h"
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
// block w/4 and the steps w%4, w%4 + 4, ... of the whole K, so the two waves
// of a step lane work on the same steps and share one L1^T slice.  Round j
// computes steps 4j .. 4j+3 (one per step lane).  The workgroup is bound by
// how many bytes it keeps in flight (a copy takes a few us under a full-chip
// load), so the ring has four LDS slots per wave (X) and per step lane
// (L1^T), three steps in flight, and runs unbroken over all of K: codes and
// scales leave from registers as each step is computed (no staging tile),
// and the reciprocals of lambda live in a double-buffered table of 2048
// channels whose next chunk is loaded during the current one.  One barrier
// per round publishes a slot and frees the oldest.  In LDS the 16-byte
// pieces of a 128-byte row segment are stored XOR-swizzled by the row (piece
// p of row i at slot p ^ ((i ^ (i >> 3)) & 7)), so the fragment reads of 16
// rows spread over the banks.
namespace dma {
constexpr int KC = 2048;  // channels per reciprocal-table chunk: 32 steps = 8 rounds
constexpr int NT = 512;
typedef __attribute__((address_space(3))) void lds_void;
typedef unsigned int u2v __attribute__((ext_vector_type(2)));

// s_waitcnt with vmcnt = n (0..63), lgkmcnt = 0, expcnt untouched
#define SVDQ_WAIT_VM_LGKM0(n) __builtin_amdgcn_s_waitcnt(((n) & 0xF) | (((n) >> 4) << 14) | 0x0070)

// the 16-byte piece p of a 128-byte row segment sits at slot p ^ rsw(row):
// rows r and r + 8 get different slots too, so a fragment read of 16 rows
// (two rows per 256 bytes of banks) touches every bank once
__device__ __forceinline__ int rsw(int row) { return (row ^ (row >> 3)) & 7; }
__device__ __forceinline__ int swz(int row, int piece) { return (piece ^ rsw(row)) << 4; }

// 16 bytes per lane, global (buffer offset off) -> LDS at dst + 16 * lane
__device__ __forceinline__ void copy16(__amdgpu_buffer_rsrc_t res, uint8_t* dst, int off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(res, (lds_void*)dst, 16, off, 0, 0, 0);
}
}  // namespace dma

// The kernel's LDS, one object so that a fused launch (quant_awq_kernel)
// can hand the same space to another job's workgroups.
template <int RB>
struct DmaLds {
  float rl[2][dma::KC];             // lambda reciprocals, two chunks
  uint8_t lst[8][1024];             // the next chunk's lambda (bf16), waves 0-3
  uint8_t xs[4][8][2048];           // X slices per ring slot and wave
  uint8_t ls[4][4][RB * 2048];      // L1^T slices per ring slot and step lane
  unsigned xflag;                   // arrival count read by the whole workgroup
};

// The body of quant_act_dma_kernel for workgroup `bid` (of a grid of the
// kernel's own size), with its LDS in S.
template <int PREC, int RB, bool CH, bool BAL>
__device__ __forceinline__ void quant_dma_body(
    DmaLds<RB>& S, int bid, int M, int K, const uint16_t* __restrict__ x, const uint16_t* __restrict__ lam,
    const uint16_t* __restrict__ l1t, float alpha, uint8_t* __restrict__ codes,
    void* __restrict__ scales, float* __restrict__ xl1, const QuantSplit& sp) {
  using namespace dma;
  static_assert(RB == 1 || RB == 2, "LDS holds L1^T slices of 16 or 32 ranks");
  constexpr int LSL = RB * 2048;    // bytes of one step's L1^T slice (16*RB rows x 128 B)
  constexpr int NDMA = 2 + RB;      // copies per wave per round: 2 for X, RB for L1^T (8 rows each)
  constexpr int NSTO = 2;           // stores per wave per round: codes, scales
  // Memory instructions retire in order and a round issues, after its
  // barrier, [the next chunk's lambda load (first round of a chunk)], the
  // copies of round j+3, then the stores of round j.  Round j needs the
  // copies of round j itself (issued three rounds earlier): what may still be
  // in flight is everything issued after them.
  constexpr int kAfter = 2 * NDMA + 3 * NSTO;
  constexpr int kOut = 0x7FFFFFF0;  // offset past num_records: zeros / dropped, no memory access
  float(&rl)[2][KC] = S.rl;
  uint8_t(&lst)[8][1024] = S.lst;
  uint8_t(*const xs0)[2048] = S.xs[0];
  uint8_t(*const xs1)[2048] = S.xs[1];
  uint8_t(*const xs2)[2048] = S.xs[2];
  uint8_t(*const xs3)[2048] = S.xs[3];
  uint8_t(*const ls0)[LSL] = S.ls[0];
  uint8_t(*const ls1)[LSL] = S.ls[1];
  uint8_t(*const ls2)[LSL] = S.ls[2];
  uint8_t(*const ls3)[LSL] = S.ls[3];
  unsigned& xflag = S.xflag;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rbk = wave >> 2, sl = wave & 3;  // row block, step lane
  const int r = lane & 15, c = lane >> 4;
  const int nsteps = K >> 6;
  // This workgroup's rounds nr (four steps each), its first 32-row block
  // pair0 and first step st0 in it, and jb, the first round in the next block
  // (past nr: none).  Balanced ranges start and end on whole rounds (L and
  // the steps per block are multiples of four), so a round never straddles
  // two blocks.
  int nr, jb, pair0, st0;
  if constexpr (BAL) {
    const int s0 = bid * sp.L;
    pair0 = s0 / nsteps;
    st0 = s0 - pair0 * nsteps;
    nr = min(sp.L, sp.T - s0) >> 2;
    jb = (nsteps - st0) >> 2;
  } else {
    pair0 = bid;
    st0 = 0;
    nr = (nsteps + 3) >> 2;
    jb = nr;
  }
  const int row0 = pair0 * 32;
  // first step (step lane 0) of round j
  auto rstep = [&](int j) __attribute__((always_inline)) -> int {
    return BAL ? (j < jb ? st0 + 4 * j : 4 * (j - jb)) : 4 * j;
  };

  const __amdgpu_buffer_rsrc_t xres = __builtin_amdgcn_make_buffer_rsrc((void*)x, (short)0, M * K * 2, 0x00020000);
  const __amdgpu_buffer_rsrc_t lres = __builtin_amdgcn_make_buffer_rsrc((void*)l1t, (short)0, RB * 16 * K * 2, 0x00020000);
  const __amdgpu_buffer_rsrc_t lamres = __builtin_amdgcn_make_buffer_rsrc((void*)lam, (short)0, lam ? K * 2 : 0, 0x00020000);
  const __amdgpu_buffer_rsrc_t cres = __builtin_amdgcn_make_buffer_rsrc((void*)codes, (short)0, M * (K >> 1), 0x00020000);
  const __amdgpu_buffer_rsrc_t sres = __builtin_amdgcn_make_buffer_rsrc(
      scales, (short)0, PREC == 0 ? M * (K >> 6) * 2 : M * (K >> 4), 0x00020000);
  // copy lanes: lane l moves piece (l%8) ^ swizzle of row l/8 of an 8-row group
  const int cr = lane >> 3;
  u32 xdo[2], ldo[RB];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int ri = 8 * i + cr;  // row within the 16-row X slice
    xdo[i] = (u32)(row0 + 16 * rbk + ri) * (u32)K * 2u + (u32)(((lane & 7) ^ rsw(ri)) << 4);
  }
#pragma unroll
  for (int i = 0; i < RB; ++i) {
    const int ri = 8 * (RB * rbk + i) + cr;  // L1^T row: this wave copies rows 8*RB*rbk .. +8*RB
    ldo[i] = (u32)ri * (u32)K * 2u + (u32)(((lane & 7) ^ rsw(ri)) << 4);
  }
  // this lane's output row and its store offsets, in the first block and (BAL)
  // the next one (rows past M: dropped)
  const int orow = row0 + 16 * rbk + r;
  const bool rlive = orow < M, rlive1 = orow + 32 < M;
  const int cbase = rlive ? orow * (K >> 1) + 8 * c : kOut;
  const int sbase = PREC == 0 ? (rlive && c == 0 ? orow * (K >> 6) * 2 : kOut) : (rlive ? orow * (K >> 4) + c : kOut);
  const int cbase1 = BAL && rlive1 ? (orow + 32) * (K >> 1) + 8 * c : kOut;
  const int sbase1 = !BAL ? kOut
                     : PREC == 0 ? (rlive1 && c == 0 ? (orow + 32) * (K >> 6) * 2 : kOut)
                                 : (rlive1 ? (orow + 32) * (K >> 4) + c : kOut);

  v4f acc[RB], accA[RB];  // accA: the first block's sums once round jb starts the next
#pragma unroll
  for (int i = 0; i < RB; ++i) acc[i] = accA[i] = v4f{0.f, 0.f, 0.f, 0.f};
  const float d6 = 6.0f * alpha;

  // copy the step of round j for this wave into slot buffers (xb, lb); steps
  // past the end use out-of-range offsets (zeros, no memory access), so every
  // wave issues the same copies in every round and the waits count exactly
  auto issue = [&](int j, uint8_t(*xb)[2048], uint8_t(*lb)[LSL]) __attribute__((always_inline)) {
    const int st = rstep(j) + sl;
    const bool live = BAL ? j < nr : st < nsteps;
    const u32 sb = 128u * (u32)st;
    const u32 xsb = sb + (BAL && j >= jb ? 64u * (u32)K : 0u);  // the next block: 32 rows further
#pragma unroll
    for (int i = 0; i < 2; ++i) copy16(xres, xb[wave] + 1024 * i, live ? (int)(xdo[i] + xsb) : kOut);
#pragma unroll
    for (int i = 0; i < RB; ++i) copy16(lres, lb[sl] + 1024 * (RB * rbk + i), live ? (int)(ldo[i] + sb) : kOut);
  };
  // the NSTO stores of a round, issued also for steps past the end (dropped)
  // (dead: the out-of-range offset of a dropped store; distinct ones keep the
  // compiler from merging the prologue's dropped stores into one)
  auto store = [&](bool live, int cb, int sbs, int st, u32 pk0, u32 pk1, u32 sbits, int dead = kOut)
      __attribute__((always_inline)) {
    __builtin_amdgcn_raw_buffer_store_b64(u2v{pk0, pk1}, cres, live ? cb + 32 * st : dead, 0, 0);
    if constexpr (PREC == 0)
      __builtin_amdgcn_raw_buffer_store_b16((unsigned short)sbits, sres, live ? sbs + 2 * st : dead, 0, 0);
    else
      __builtin_amdgcn_raw_buffer_store_b8((unsigned char)sbits, sres, live ? sbs + 4 * st : dead, 0, 0);
  };
  // lambda of a chunk: thread t < 256 loads channels 8t .. 8t+7 (16 bytes);
  // for the first chunk straight into registers, for the next ones by a copy
  // into lst (a register load issued rounds before its use would be sunk by
  // the compiler to its use, stalling the ring there), one per wave
  auto lam_load = [&](int q) __attribute__((always_inline)) -> uint4 {
    const int ch = q * KC + 8 * tid;
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                         lamres, tid < KC / 8 && ch < K ? 2 * ch : kOut, 0, 0));
  };
  auto lam_copy = [&](int q) __attribute__((always_inline)) {
    const int ch = q * KC + 8 * tid;
    copy16(lamres, lst[wave], wave < 4 && ch < K ? 2 * ch : kOut);
  };
  // reciprocals of the eight lambda values in lv, to dst[0 .. 8)
  auto lam_recip = [&](float* dst, uint4 lv) __attribute__((always_inline)) {
    const u32 w4[4] = {lv.x, lv.y, lv.z, lv.w};
    float o[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      o[2 * e] = lam ? 1.0f / bf16_bits_to_f32(w4[e] & 0xFFFFu) : 1.0f;
      o[2 * e + 1] = lam ? 1.0f / bf16_bits_to_f32(w4[e] >> 16) : 1.0f;
    }
    *(float4*)dst = float4{o[0], o[1], o[2], o[3]};
    *(float4*)(dst + 4) = float4{o[4], o[5], o[6], o[7]};
  };

  // quantize the step of round j from slot buffers (xb, lb), store its codes
  // and scale, and add its X.L1 share
  auto compute = [&](int j, uint8_t(*xb)[2048], uint8_t(*lb)[LSL]) __attribute__((always_inline)) {
    const int st = rstep(j) + sl;  // step within K
    const bool nxt = BAL && j >= jb;
    // a chunked table holds the chunk of rounds 8t .. 8t+7 in buffer t & 1
    const float* rlc = CH ? &rl[(j >> 3) & 1][((st & 31) << 6) + (c << 4)] : &rl[0][0] + (st << 6) + (c << 4);
    const uint8_t* xrow = xb[wave] + r * 128;
    const uint4 va = *(const uint4*)(xrow + swz(r, 2 * c));
    const uint4 vb = *(const uint4*)(xrow + swz(r, 2 * c + 1));
    const u32 xw[8] = {va.x, va.y, va.z, va.w, vb.x, vb.y, vb.z, vb.w};
    float rk[16];
    *(float4*)&rk[0] = *(const float4*)&rlc[0];
    *(float4*)&rk[4] = *(const float4*)&rlc[4];
    *(float4*)&rk[8] = *(const float4*)&rlc[8];
    *(float4*)&rk[12] = *(const float4*)&rlc[12];
    float xh[16];
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      xh[2 * i] = bf16_bits_to_f32(xw[i] & 0xFFFFu) * rk[2 * i];
      xh[2 * i + 1] = bf16_bits_to_f32(xw[i] >> 16) * rk[2 * i + 1];
      amax = fmaxf(amax, fmaxf(fabsf(xh[2 * i]), fabsf(xh[2 * i + 1])));
    }
    u32 pk0, pk1, sbits;
    if constexpr (PREC == 0) {
      amax = max_over_rows(amax);  // one 64-channel group = lanes l, l^16, l^32, l^48
      sbits = f32_to_f16_sat_bits(div7_rn(amax));
      const float sf = f16_bits_to_f32(sbits);
      const float t = sf == 0.0f ? 0.0f : 1.0f / sf;
      pk0 = int4_codes8(xh, t);
      pk1 = int4_codes8(xh + 8, t);
    } else {
      // one 16-channel group = this lane's 16 channels
      sbits = f32_to_e4m3_sat_pos(amax / d6);
      const float sf = e4m3_to_f32(sbits);
      float t = 0.0f;
      if (sf != 0.0f) {
        const float sa = sf * alpha;
        t = 1.0f / sa;
      }
      // a zero scale writes code 0 (t = 0 would give -0 codes for negative xh)
      pk0 = sf == 0.0f ? 0u : e2m1_codes8(xh, t);
      pk1 = sf == 0.0f ? 0u : e2m1_codes8(xh + 8, t);
    }
    store(BAL ? j < nr : st < nsteps, nxt ? cbase1 : cbase, nxt ? sbase1 : sbase, st, pk0, pk1, sbits);
    if constexpr (BAL) {
      if (j == jb && j < nr) {  // first round of the next block: set the first block's sums aside
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          accA[rb] = acc[rb];
          acc[rb] = v4f{0.f, 0.f, 0.f, 0.f};
        }
      }
    }
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
  };

  // Prologue: the load of lambda (the whole table for K <= 2 KC, else the
  // first chunk) goes out first, then rounds 0 .. 2, each followed by NSTO
  // dropped stores so that every later round finds the same instruction
  // pattern behind its copies (the waits below count it); the reciprocals are
  // formed once lambda has landed, while the copies are still in flight.
  uint4 lv0;
  if constexpr (CH) {
    lv0 = lam_load(rstep(0) >> 5);
  } else {
    const int ch = 8 * tid;
    lv0 = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(lamres, ch < K ? 2 * ch : kOut, 0, 0));
  }
  // The round waits count memory instructions, so all three pairs of dropped
  // stores must be emitted, each after its copies: they go to distinct
  // out-of-range offsets (identical ones were merged into one pair, which left
  // round 0's wait short of round 0's copies) and each group is fenced.
  // tests/test_quant_asm.py checks the emitted order in the gfx950 assembly.
  asm volatile("" ::: "memory");
  issue(0, xs0, ls0);
  store(false, cbase, sbase, 0, 0u, 0u, 0u, kOut);
  asm volatile("" ::: "memory");
  issue(1, xs1, ls1);
  store(false, cbase, sbase, 0, 0u, 0u, 0u, kOut - 256);
  asm volatile("" ::: "memory");
  issue(2, xs2, ls2);
  store(false, cbase, sbase, 0, 0u, 0u, 0u, kOut - 512);
  asm volatile("" ::: "memory");
  if constexpr (CH) {
    if (tid < KC / 8) lam_recip(&rl[0][8 * tid], lv0);
  } else {
    lam_recip(&rl[0][0] + 8 * tid, lv0);
  }

  // Round j = 8t + P: wait for this wave's copies of round j and its LDS
  // traffic, barrier (every wave's copies of round j have landed; every wave
  // is done with the slot of round j-1 and, at P = 0, with the reciprocal
  // buffer of the chunk before), then, with a chunked table, at P = 0 copy
  // the chunk of round j+8 (landed by the wait of round j+3, where the table
  // is filled; lst is rewritten only by the next chunk's P = 0, after that
  // round's barrier), refill the freed slot with round j+3, compute round j.
  // Steps past the end (the rounds that pad the loop to whole unrolled
  // blocks, before the exit test stops it) are computed on the zeros their
  // copies brought and their stores dropped: no branch inside a round, so the
  // compiler keeps track of which copy fills which slot and adds no waits of
  // its own.
  auto round = [&](int j, auto pc, uint8_t(*xa)[2048], uint8_t(*la)[LSL], uint8_t(*xc)[2048], uint8_t(*lc)[LSL])
      __attribute__((always_inline)) {
    constexpr int P = decltype(pc)::value;
    SVDQ_WAIT_VM_LGKM0(kAfter + (CH && (P == 1 || P == 2) ? 1 : 0));
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if constexpr (CH && P == 0) lam_copy(rstep(j + 8) >> 5);
    issue(j + 3, xc, lc);
    if constexpr (CH && P == 3) {
      if (tid < KC / 8) lam_recip(&rl[((j >> 3) + 1) & 1][8 * tid], *(const uint4*)&lst[tid >> 6][16 * (tid & 63)]);
    }
    compute(j, xa, la);
  };
  using P0 = std::integral_constant<int, 0>;
  using P1 = std::integral_constant<int, 1>;
  using P2 = std::integral_constant<int, 2>;
  using P3 = std::integral_constant<int, 3>;
  using P4 = std::integral_constant<int, 4>;
  using P5 = std::integral_constant<int, 5>;
  using P6 = std::integral_constant<int, 6>;
  using P7 = std::integral_constant<int, 7>;
  if constexpr (CH) {
    for (int j = 0; j < nr; j += 8) {
      round(j, P0{}, xs0, ls0, xs3, ls3);
      if (j + 1 >= nr) break;
      round(j + 1, P1{}, xs1, ls1, xs0, ls0);
      if (j + 2 >= nr) break;
      round(j + 2, P2{}, xs2, ls2, xs1, ls1);
      if (j + 3 >= nr) break;
      round(j + 3, P3{}, xs3, ls3, xs2, ls2);
      if (j + 4 >= nr) break;
      round(j + 4, P4{}, xs0, ls0, xs3, ls3);
      if (j + 5 >= nr) break;
      round(j + 5, P5{}, xs1, ls1, xs0, ls0);
      if (j + 6 >= nr) break;
      round(j + 6, P6{}, xs2, ls2, xs1, ls1);
      if (j + 7 >= nr) break;
      round(j + 7, P7{}, xs3, ls3, xs2, ls2);
    }
  } else {
    for (int j = 0; j < nr; j += 4) {
      round(j, P4{}, xs0, ls0, xs3, ls3);
      if (j + 1 >= nr) break;
      round(j + 1, P5{}, xs1, ls1, xs0, ls0);
      if (j + 2 >= nr) break;
      round(j + 2, P6{}, xs2, ls2, xs1, ls1);
      if (j + 3 >= nr) break;
      round(j + 3, P7{}, xs3, ls3, xs2, ls2);
    }
  }

  // per-wave partial XL1 tiles [16 rows][R] in slot xs0 (every copy has
  // landed and every wave is past its last read), summed over the four step
  // lanes of each row block in a fixed order; lane holds
  // D[row 4*(lane/16) + v][col lane%16] of each 16x16 block.  Thread t ends
  // with the sums of tile entries t + NT k (row (t + NT k) / R), k < RB.
  constexpr int R = RB * 16;
  constexpr int TILE = 32 * R;
  static_assert(TILE == RB * NT, "RB tile entries per thread");
  __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0), lgkmcnt(0)
  __syncthreads();
  float* red = (float*)&xs0[0][0];
  static_assert(8 * 16 * R * 4 <= 8 * 2048, "partial XL1 tiles fit in one X slot");
  float sums[RB];
  auto reduce = [&](const v4f* a) __attribute__((always_inline)) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int v = 0; v < 4; ++v) red[(wave * 16 + 4 * c + v) * R + rb * 16 + r] = a[rb][v];
    __syncthreads();
#pragma unroll
    for (int k = 0; k < RB; ++k) {
      const int idx = tid + NT * k;
      const int rr = idx / R, col = idx - rr * R;  // row within the 32
      const int b = rr >> 4, ri = rr & 15;
      float sum = red[((4 * b) * 16 + ri) * R + col];
#pragma unroll
      for (int s2 = 1; s2 < 4; ++s2) sum += red[((4 * b + s2) * 16 + ri) * R + col];  // fixed order
      sums[k] = sum;
    }
  };
  auto write_rows = [&](int rbase, const float* s) __attribute__((always_inline)) {
#pragma unroll
    for (int k = 0; k < RB; ++k) {
      const int idx = tid + NT * k;
      const int rr = idx / R;
      if (rbase + rr < M) xl1[(size_t)rbase * R + idx] = s[k];
    }
  };
  if constexpr (!BAL) {
    reduce(acc);
    write_rows(row0, sums);
  } else {
    // A block shared with other workgroups: store this piece's tile with
    // agent-coherent stores, wait until they are performed, count the piece
    // in; the last piece to arrive resets the counter and writes the block's
    // XL1 as the sum of all pieces in workgroup order (the same sum whichever
    // arrives last).  No workgroup waits for another.
    auto exchange = [&](int p, int seg) __attribute__((always_inline)) {
      const int first = (int)(((long long)p * nsteps) / sp.L);
      const int last = (int)(((long long)(p + 1) * nsteps - 1) / sp.L);
      float* const mine = sp.part + (size_t)(2 * bid + seg) * TILE;
#pragma unroll
      for (int k = 0; k < RB; ++k) __hip_atomic_store(mine + tid + NT * k, sums[k], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      __builtin_amdgcn_s_waitcnt(0);  // every store of this wave performed
      __syncthreads();
      if (tid == 0) xflag = __hip_atomic_fetch_add(sp.cnt + first, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __syncthreads();
      const unsigned arrived = __builtin_amdgcn_readfirstlane(*(volatile unsigned*)&xflag);
      if (arrived != (unsigned)(last - first)) return;
      if (tid == 0) __hip_atomic_store(sp.cnt + first, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      float tot[RB];
#pragma unroll
      for (int k = 0; k < RB; ++k) tot[k] = 0.0f;
      for (int w = first; w <= last; ++w) {
        const int slot = 2 * w + (p - (int)(((long long)w * sp.L) / nsteps));
        const float* src = sp.part + (size_t)slot * TILE;
#pragma unroll
        for (int k = 0; k < RB; ++k)
          tot[k] += w == bid ? sums[k]
                                         : __hip_atomic_load(src + tid + NT * k, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      write_rows(p * 32, tot);
    };
    const bool two = jb < nr;
    if (two) reduce(accA);
    else reduce(acc);
    if (st0 == 0 && nr >= jb) write_rows(row0, sums);  // the whole block is this workgroup's
    else exchange(pair0, 0);
    if (two) {
      __syncthreads();  // every wave is done with red and xflag
      reduce(acc);
      exchange(pair0 + 1, 1);
    }
  }
}

template <int PREC, int RB, bool CH, bool BAL>
__global__ __launch_bounds__(dma::NT) void quant_act_dma_kernel(
    int M, int K, const uint16_t* __restrict__ x, const uint16_t* __restrict__ lam,
    const uint16_t* __restrict__ l1t, float alpha, uint8_t* __restrict__ codes,
    void* __restrict__ scales, float* __restrict__ xl1, QuantSplit sp) {
  __shared__ __align__(16) DmaLds<RB> S;
  quant_dma_body<PREC, RB, CH, BAL>(S, (int)blockIdx.x, M, K, x, lam, l1t, alpha, codes, scales, xl1, sp);
}

template <int PREC, int RB, bool CH, bool BAL>
static hipError_t launch_dma(const QuantArgs& a, int blocks, const QuantSplit& sp, hipStream_t st) {
  hipLaunchKernelGGL((quant_act_dma_kernel<PREC, RB, CH, BAL>), dim3(blocks), dim3(dma::NT), 0, st, (int)a.M,
                     (int)a.K, (const uint16_t*)a.x, (const uint16_t*)a.smooth, (const uint16_t*)a.l1t, a.alpha,
                     (uint8_t*)a.codes, a.scales, a.xl1, sp);
  return hipGetLastError();
}

// The balanced split of svdq_quantize_act_ws: ranges of L steps, L the even
// share of the CUs rounded up to whole rounds (whole 2048-channel chunks of
// the reciprocal table when K > 2 KC), used when the blocks' steps are whole
// such units and the split saves at least eight of a block's rounds (32
// steps): it costs a few rounds' time in the exchange of the shared blocks'
// XL1 and in the larger number of workgroups copying at once (measured by
// kernel trace on a 4608 x 3072 input, where it saves five: 14.9 us against
// 13.8 us unsplit).  Returns false (sp untouched) where it does not apply.
static bool balanced_split(const QuantArgs& a, QuantSplit& sp, int& blocks) {
  if (!a.work || a.M <= 0) return false;
  const int nsteps = (int)(a.K >> 6);
  const int unit = a.K > 2 * dma::KC ? 32 : 4;
  if (nsteps % unit != 0) return false;
  const long long T = (long long)((a.M + 31) / 32) * nsteps;
  const int cus = device_cu_count();
  long long L = (T + cus - 1) / cus;
  L = (L + unit - 1) / unit * unit;
  if (nsteps - L < 32) return false;
  const long long G = (T + L - 1) / L;
  if (G > kQuantMaxGroups) return false;
  sp.L = (int)L;
  sp.T = (int)T;
  sp.part = (float*)a.work;
  sp.cnt = (unsigned*)((uint8_t*)a.work + kQuantCntOffset);
  blocks = (int)G;
  return true;
}

template <int PREC, int RB>
static hipError_t launch_quant_dma(const QuantArgs& a, hipStream_t st) {
  QuantSplit sp{0, 0, nullptr, nullptr};
  int blocks = (int)((a.M + 31) / 32);
  const bool ch = a.K > 2 * dma::KC;  // else the whole reciprocal table in LDS
  if (balanced_split(a, sp, blocks))
    return ch ? launch_dma<PREC, RB, true, true>(a, blocks, sp, st) : launch_dma<PREC, RB, false, true>(a, blocks, sp, st);
  return ch ? launch_dma<PREC, RB, true, false>(a, blocks, sp, st) : launch_dma<PREC, RB, false, false>(a, blocks, sp, st);
}

template <int PREC, int RB>
static hipError_t launch_quant(const QuantArgs& a, hipStream_t st) {
  // Ranks 16 / 32: once the 16-row workgroups of the kernel above no longer
  // fit one per CU, the LDS-staged kernel (32 rows per workgroup, coalesced
  // copies) is faster, for both precisions; below that the one-row-block
  // workgroups keep every CU busy.  With a workspace, the LDS-staged kernel's
  // balanced split applies at any M where it cuts the work per CU.
  if constexpr (RB == 1 || RB == 2) {
    QuantSplit sp{0, 0, nullptr, nullptr};
    int blocks = 0;
    if ((a.M + 15) / 16 > device_cu_count() || balanced_split(a, sp, blocks)) return launch_quant_dma<PREC, RB>(a, st);
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

// One launch of two independent jobs (svdq_quantize_act_awq_gemv): workgroups
// [0, qblocks) run the LDS-staged quantizer exactly as quant_act_dma_kernel
// (unsplit), the others the small-M AWQ GEMV with eight waves (awq_gemv_body,
// 32 weight rows per workgroup) in the same LDS.  On a DiT-sized call the
// quantizer's 32-row workgroups hold one CU each and leave the rest idle (144
// of 256 CUs at 4608 rows) for ~15 us; the GEMV's workgroups, dispatched after
// them, stream the 4-bit weights there meanwhile, and its own launch, ramp
// and tail are gone.  Each job computes what its own launch computes.
template <int PREC, int RB, int MR, int SX>
__global__ __launch_bounds__(dma::NT) void quant_awq_kernel(
    int qblocks, int M, int K, const uint16_t* __restrict__ x, const uint16_t* __restrict__ lam,
    const uint16_t* __restrict__ l1t, float alpha, uint8_t* __restrict__ codes, void* __restrict__ scales,
    float* __restrict__ xl1, int aM, int aN, int aK, const uint16_t* __restrict__ ax,
    const uint8_t* __restrict__ wc, const uint16_t* __restrict__ ws, const uint16_t* __restrict__ wz,
    const uint16_t* __restrict__ bias, uint16_t* __restrict__ ay) {
  static_assert(dma::NT == 64 * 8, "the GEMV's workgroups take the quantizer's eight waves");
  __shared__ __align__(16) DmaLds<RB> S;
  const int b = (int)blockIdx.x;
  if (b < qblocks) {
    const QuantSplit none{0, 0, nullptr, nullptr};
    quant_dma_body<PREC, RB, false, false>(S, b, M, K, x, lam, l1t, alpha, codes, scales, xl1, none);
  } else {
    awq_gemv_body<MR, SX, 8>((uint4*)&S, b - qblocks, aM, aN, aK, ax, wc, ws, wz, bias, ay);
  }
}

namespace {
// The fused launch applies where each job would take that kernel on its own
// launch: the quantizer's LDS-staged kernel with one reciprocal table and no
// split (ranks 16 and 32, more 16-row blocks than CUs, K <= 4096), and the
// small-M GEMV (M <= 4, K % 512 == 0, K <= 8192) with eight-wave workgroups
// (N % 32 == 0) whose LDS fits the quantizer's.
template <int PREC, int RB, int MR>
hipError_t launch_quant_awq_sx(const QuantArgs& q, const AwqArgs& w, int sx, hipStream_t st) {
  typedef void (*F)(int, int, int, const uint16_t*, const uint16_t*, const uint16_t*, float, uint8_t*, void*, float*,
                    int, int, int, const uint16_t*, const uint8_t*, const uint16_t*, const uint16_t*,
                    const uint16_t*, uint16_t*);
  static const F table[4] = {quant_awq_kernel<PREC, RB, MR, 1>, quant_awq_kernel<PREC, RB, MR, 2>,
                             quant_awq_kernel<PREC, RB, MR, 4>, quant_awq_kernel<PREC, RB, MR, 8>};
  const int si = sx <= 1 ? 0 : sx <= 2 ? 1 : sx <= 4 ? 2 : 3;
  const int qblocks = (int)((q.M + 31) / 32);
  const int ablocks = (int)(w.N / 32);
  hipLaunchKernelGGL(table[si], dim3(qblocks + ablocks), dim3(dma::NT), 0, st, qblocks, (int)q.M, (int)q.K,
                     (const uint16_t*)q.x, (const uint16_t*)q.smooth, (const uint16_t*)q.l1t, q.alpha,
                     (uint8_t*)q.codes, q.scales, q.xl1, (int)w.M, (int)w.N, (int)w.K, (const uint16_t*)w.x,
                     (const uint8_t*)w.w_codes, (const uint16_t*)w.w_scales, (const uint16_t*)w.w_zeros,
                     (const uint16_t*)w.bias, (uint16_t*)w.y);
  return hipGetLastError();
}

template <int PREC, int RB>
hipError_t launch_quant_awq_mr(const QuantArgs& q, const AwqArgs& w, int sx, hipStream_t st) {
  return w.M <= 1 ? launch_quant_awq_sx<PREC, RB, 1>(q, w, sx, st)
       : w.M <= 2 ? launch_quant_awq_sx<PREC, RB, 2>(q, w, sx, st)
                  : launch_quant_awq_sx<PREC, RB, 4>(q, w, sx, st);
}
}  // namespace

bool quant_awq_fusable(const QuantArgs& q, const AwqArgs& w, int* sx) {
  if (q.M <= 0 || w.M <= 0) return false;
  if (!(q.rank == 16 || q.rank == 32) || (q.M + 15) / 16 <= device_cu_count() || q.K > 2 * dma::KC) return false;
  if (w.M > 4 || w.K % 512 != 0 || w.K / 512 > AWQ_TBMAX || w.N % 32 != 0) return false;
  const int MR = w.M <= 1 ? 1 : w.M <= 2 ? 2 : 4;
  const AwqLds L = awq_lds((int)w.K, MR, 32);
  const int items = (L.nx + dma::NT - 1) / dma::NT;  // x staging items per thread
  const size_t lds = q.rank == 16 ? sizeof(DmaLds<1>) : sizeof(DmaLds<2>);
  if ((size_t)L.total > lds || items > 8) return false;
  *sx = items;
  return true;
}

hipError_t launch_quant_awq(const QuantArgs* q, const AwqArgs* w, hipStream_t st) {
  int sx = 0;
  if (q && w && quant_awq_fusable(*q, *w, &sx)) {
    const bool r16 = q->rank == 16;
    if (q->precision == 0)
      return r16 ? launch_quant_awq_mr<0, 1>(*q, *w, sx, st) : launch_quant_awq_mr<0, 2>(*q, *w, sx, st);
    return r16 ? launch_quant_awq_mr<1, 1>(*q, *w, sx, st) : launch_quant_awq_mr<1, 2>(*q, *w, sx, st);
  }
  if (q) {
    const hipError_t e = launch_quantize_act(*q, st);
    if (e != hipSuccess) return e;
  }
  return w ? launch_awq(*w, st) : hipSuccess;
}

}  // namespace svdq
