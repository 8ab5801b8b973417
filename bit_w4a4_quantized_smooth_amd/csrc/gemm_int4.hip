// W4A4 int4 GEMM of the SVDQuant linear with per-group dequantization and the
// low-rank up-projection and bias fused into the epilogue (blog "Nunchaku
// 4-bit inference in Diffusers", "Background: SVDQuant and Nunchaku"; int4 /
// group 64 from "Nunchaku Lite", "Supported quantization types").
//
//   y[m,n] = sum_g sa[m,g] * sw[n,g] * P[m,n,g] + sum_j XL1[m,j] L2[j,n] + bias[n]
//   P[m,n,g] = sum_{k in g} qa[m,k] * qw[n,k]                    (exact int32)
//
// gfx950 design
// -------------
// * Workgroup = 4 wave64 (2x2) computing a 128(n) x 128(m) tile of Y^T; each
//   wave owns 64x64 = 4x4 blocks of 16x16.  The matrix-core A operand is the
//   weight tile (rows n) and B the activation tile (columns m).  Two
//   workgroups share a CU.
// * Two 64-channel groups per double-buffered LDS stage: each row contributes
//   a 64-byte segment of packed codes (four 16-byte loads per row).  While
//   staging to LDS the nibbles are expanded to int8 16*q: the two's
//   complement nibble in the high half of a byte is 16*q exactly (one mask
//   for odd channels, one shift and mask for even ones, no sign extension).
//   The 16-byte pieces of a 128-byte LDS row are XOR-swizzled by the row
//   (piece p of row r at p ^ (r & 7)), so rows need no padding.
//   Both operands get the same channel permutation, so P is unchanged and the
//   matrix core (v_mfma_i32_16x16x64_i8, one per block and group) returns
//   256*P.
// * int32 -> fp32 without a conversion instruction: each group's product
//   starts from the accumulator bit pattern of c0 = 1/(2 pi) (an inline
//   constant), whose mantissa leaves more than 2^20 of head-room on both
//   sides; the integer sum bits(c0) + 256*P is therefore the float
//   c0 + P*2^-18 exactly.
// * The per-group scale product S = sw (x) sa is an outer product computed on
//   the matrix core by v_mfma_f32_16x16x4_4b_f16 (four independent 16x16
//   blocks; each lane gives its fp16 scale as k = 0 and zeros for k = 1..3, so
//   the fp32 result is the exact product of the two fp16 scales: a 2x2 quad
//   of output blocks), leaving one VALU FMA per output per group: acc += S *
//   (c0 + P*2^-18).  The fp16 instruction runs beside the vector ALU, where
//   the fp32 outer product (v_mfma_f32_16x16x1_4b_f32) stalls it: 4-5% on
//   every shape, results identical.  Quads are software
//   pipelined: the FMAs of quad Q-1 issue under the five matrix instructions
//   of quad Q.  The epilogue removes the constant: y = 2^18 * (acc - c0 *
//   sum_g S), where sum_g S = Sw . Sa^T is one small K = #groups fp16 GEMM on
//   the matrix core (fp16 x fp16 products are exact in fp32).
// * Operand loads are raw buffer loads: rows past the end of a tensor read as
//   zero in hardware, so the M and N tails need no per-lane predication.
// * Tiles are ordered so that each XCD (own L2) works on a contiguous range
//   of a banded order: the tiles resident on one XCD at a time share a few
//   activation and weight panels in that XCD's L2.
#include <atomic>
#include <type_traits>

#include "common.h"
#include "launch.h"
#include "mlp_epi.h"
#include "qkv_epi.h"
#include "tail_split.h"

namespace svdq {

typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef float v32f __attribute__((ext_vector_type(32)));
typedef _Float16 v4h __attribute__((ext_vector_type(4)));
typedef __bf16 v4bf __attribute__((ext_vector_type(4)));

// Tile configuration: WAVES_N x WAVES_M waves, each owning a (16*BI) x (16*BJ)
// tile of 16x16 blocks; KG 64-channel groups per pipeline stage.
constexpr int WAVES_N = 2, WAVES_M = 2, BI = 4, BJ = 4, KG = 2;

namespace {
constexpr int BN = WAVES_N * BI * 16, BM = WAVES_M * BJ * 16;
constexpr int NT = WAVES_N * WAVES_M * 64;
constexpr int PARTS = 2 * KG;                       // 16-byte code parts per row per stage
constexpr int ROWB = 64 * KG;                       // LDS bytes per operand row (int8), pieces swizzled
constexpr int NROWS = BN + BM;                      // W rows then X rows in one LDS stage
constexpr int CHUNKS = NROWS * PARTS / NT;          // 16-byte loads per thread per stage
constexpr int SROWS = (NROWS + NT - 1) / NT;        // scale rows per thread
constexpr int STAGE = NROWS * ROWB;                 // bytes of one stage of operands
constexpr int SC_STAGE = NROWS * KG;                // scale operands (8 bytes each) of one stage
constexpr size_t LDS_BYTES = 2 * (size_t)STAGE + 2 * (size_t)SC_STAGE * 8;
// The integer accumulator starts from the bit pattern of the fp32 number
// c0 = 0x3E22F983 (the inline constant 1/(2 pi)), whose mantissa leaves more
// than 2^20 of head-room on both sides: the integer sum c0_bits + 256*P is the
// float c0 + P * 2^-18 exactly (|256 P| <= 2^20).
constexpr int kMagicBits = 0x3E22F983;
constexpr float kMagicScale = 262144.0f;            // 2^18
constexpr uint32_t kBufDword3 = 0x00020000u;        // raw buffer, 32-bit data format
static_assert(NROWS * PARTS % NT == 0, "stage loads must divide evenly");
static_assert(BN % 128 == 0, "weight tile in halves of 128 rows");
static_assert(BI % 2 == 0 && BJ % 2 == 0, "scale outer products cover 2x2 quads of blocks");
static_assert((NT / 64) * BI * BJ * 64 * 16 <= LDS_BYTES, "K-split accumulator exchange fits a copy's LDS");
static_assert(2 * LDS_BYTES <= 160 * 1024, "K-split workgroup fits the CU's LDS");

__device__ __forceinline__ uint4 nib_lo16(uint4 v) {  // 16*q of even channels
  return uint4{(v.x << 4) & 0xF0F0F0F0u, (v.y << 4) & 0xF0F0F0F0u, (v.z << 4) & 0xF0F0F0F0u,
               (v.w << 4) & 0xF0F0F0F0u};
}
__device__ __forceinline__ uint4 nib_hi16(uint4 v) {  // 16*q of odd channels
  return uint4{v.x & 0xF0F0F0F0u, v.y & 0xF0F0F0F0u, v.z & 0xF0F0F0F0u, v.w & 0xF0F0F0F0u};
}

}  // namespace

// MODE 0: Y = bf16 linear output; 1: int32 partial products; 2: Y of the fused
// attention projection (Q/K RMSNorm and rotary embedding in the epilogue);
// 3: fused MLP up-projection (no Y: GELU, then the down projection's
// quantization and low-rank input)
//
// SPLIT 2 (plain GEMM only): 2 NT threads per tile; threads [NT, 2 NT) are a
// second copy of the workgroup that stages and multiplies the second half of
// the K range in LDS of its own, and hands its fp32 accumulators to the first
// copy through LDS before the epilogue.  A tile that has a CU to itself (grids
// of at most one tile per CU) runs its chain of group products as two chains
// of half the length on two waves per SIMD.
template <int MODE, bool SCD, int SPLIT>
__global__ __launch_bounds__(NT * SPLIT, 1) void gemm_int4_kernel(
    int M, int N, int K, int rank, const uint8_t* __restrict__ ac, const uint16_t* __restrict__ as,
    const uint8_t* __restrict__ wc, const uint16_t* __restrict__ ws, const float* __restrict__ xl1,
    const uint16_t* __restrict__ l2t, const uint16_t* __restrict__ bias, uint16_t* __restrict__ y,
    int32_t* __restrict__ psums, QkvEpi qe, MlpEpi me, TailSplit ts) {
  static_assert(SPLIT == 1 || (SPLIT == 2 && MODE == 0), "K split only for the plain GEMM");
  extern __shared__ __align__(16) uint8_t smem[];
  const int half = SPLIT == 2 ? __builtin_amdgcn_readfirstlane((int)threadIdx.x / NT) : 0;
  uint8_t* const sm = smem + half * LDS_BYTES;  // this copy's staging LDS
  // [2][KG][NROWS] scales, each as the 8 bytes (fp16 bits, 0, 0, 0): the
  // (scale, 0, 0, 0) operand of the 4-block scale product, read as is
  uint2* ssc = (uint2*)(sm + 2 * STAGE);

  const int tid = (int)threadIdx.x & (NT - 1), wave = tid >> 6, lane = tid & 63;
  const int l16 = lane & 15, lg = lane >> 4;  // lane within a 16-lane group, group 0..3

  // Tile order.  Consecutive workgroup ids go round-robin over the 8 XCDs
  // (each with its own L2): first give each XCD a contiguous range of the
  // order, then walk the tile grid in bands of kBandM row tiles (m fastest
  // inside a band), so the tiles an XCD runs at once share a few activation
  // and weight panels that fit its L2 instead of sweeping all of M per column.
  const int m_tiles = (M + BM - 1) / BM, n_tiles = (N + BN - 1) / BN;  // N % 128 == 0
  const int tiles = m_tiles * n_tiles;
  int t = blockIdx.x;
  // A K slice of a tile of the last partial round (plain GEMM, grid split by
  // the launcher): its tile is one of the last tail/8 of its XCD's range, so
  // every slice of a tile runs on the same XCD as the tile's neighbours.
  int slice = -1, tail_idx = 0;
  constexpr bool kTailSplit = (MODE == 0 || MODE == 2) && SPLIT == 1;  // the Y-producing GEMMs
  if ((tiles & 7) == 0) t = split_tile_of(t, tiles, kTailSplit ? ts : TailSplit{}, slice, tail_idx);
  constexpr int kBandM = 12;
  const int band = t / (kBandM * n_tiles), in_band = t - band * (kBandM * n_tiles);
  const int band_m0 = band * kBandM;
  const int band_h = m_tiles - band_m0 < kBandM ? m_tiles - band_m0 : kBandM;
  const int m0 = (band_m0 + in_band % band_h) * BM, n0 = (in_band / band_h) * BN;
  const int wn = (wave / WAVES_M) * (BI * 16), wm = (wave % WAVES_M) * (BJ * 16);
  const int G = K >> 6;
  const int stages = (G + KG - 1) / KG;
  int lstages = stages / SPLIT;  // stages of this copy (SPLIT divides stages)
  int s_off = half * lstages;    // its first stage
  if (kTailSplit && slice >= 0) {  // slice p: stages [p*stages/parts, (p+1)*stages/parts)
    s_off = slice * stages / ts.parts;
    lstages = (slice + 1) * stages / ts.parts - s_off;
  }
  const int rowb = K >> 1;

  // Buffer resources: reads past the last row return zeros (the M and N tails).
  const __amdgpu_buffer_rsrc_t wres = __builtin_amdgcn_make_buffer_rsrc((void*)wc, (short)0, N * rowb, kBufDword3);
  const __amdgpu_buffer_rsrc_t xres = __builtin_amdgcn_make_buffer_rsrc((void*)ac, (short)0, M * rowb, kBufDword3);
  const __amdgpu_buffer_rsrc_t wsres = __builtin_amdgcn_make_buffer_rsrc((void*)ws, (short)0, MODE != 1 ? N * G * 2 : 0, kBufDword3);
  const __amdgpu_buffer_rsrc_t asres = __builtin_amdgcn_make_buffer_rsrc((void*)as, (short)0, MODE != 1 ? M * G * 2 : 0, kBufDword3);

  // staging: chunk c = tid + NT*r -> (row c / PARTS, 16-byte part c % PARTS);
  // rows [0, BN) are weight rows n0+row, rows [BN, NROWS) activation rows.
  // Chunks r < WCH hold weight rows for every thread (NT % PARTS == 0), so the
  // buffer resource of each load is known at compile time.  Offsets stay in
  // the vector operand, which the hardware range-checks: a group past the end
  // of K (odd number of groups) reads the next row's bytes, or zeros past the
  // tensor; its scales are zero, so it adds nothing.
  constexpr int WCH = BN * PARTS / NT;
  static_assert(BN * PARTS % NT == 0, "weight rows fill whole chunk rounds");
  const int part = tid % PARTS;
  int coff[CHUNKS];  // byte offset of the chunk in its tensor at stage 0
#pragma unroll
  for (int r = 0; r < CHUNKS; ++r) {
    const int row = (tid + NT * r) / PARTS;
    coff[r] = r < WCH ? (n0 + row) * rowb + part * 16 : (m0 + row - BN) * rowb + part * 16;
  }
  // scale rows: row = tid + NT*r; each wave lies wholly in the weight rows or
  // in the activation rows (BN % 64 == 0), so the choice is wave-uniform
  static_assert(BN % 64 == 0, "scale rows split on a wave boundary");
  int soff[SROWS];
  bool s_is_w[SROWS], s_live[SROWS];
#pragma unroll
  for (int r = 0; r < SROWS; ++r) {
    const int row = tid + NT * r;
    const int row0 = __builtin_amdgcn_readfirstlane(row - lane);  // first row of this wave
    s_is_w[r] = row0 < BN;
    s_live[r] = row0 < NROWS;
    soff[r] = s_is_w[r] ? (n0 + row) * G * 2 : (m0 + row - BN) * G * 2;
  }

  uint4 rc[CHUNKS];
  uint32_t rs[SROWS][KG];  // raw fp16 bits: converted only at the LDS store, so
                           // no instruction waits on these loads before then
  auto gload = [&](int s) {
    const int kbyte = (s + s_off) * 32 * KG;
#pragma unroll
    for (int r = 0; r < CHUNKS; ++r)
      rc[r] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r < WCH ? wres : xres, coff[r] + kbyte, 0, 0));
    if constexpr (MODE != 1) {
      if constexpr (KG == 2 && SCD) {
        // scales come in blocks of four stages (sbload)
      } else {
#pragma unroll
        for (int r = 0; r < SROWS; ++r) {
#pragma unroll
          for (int gg = 0; gg < KG; ++gg) {
            const int g = (s + s_off) * KG + gg;
            uint32_t h = 0u;
            if (s_live[r] && g < G)  // wave-uniform
              h = s_is_w[r] ? __builtin_amdgcn_raw_buffer_load_b16(wsres, soff[r] + 2 * g, 0, 0)
                            : __builtin_amdgcn_raw_buffer_load_b16(asres, soff[r] + 2 * g, 0, 0);
            rs[r][gg] = h;
          }
        }
      }
    }
  };
  // Even group count: the fp16 scales of four stages (eight groups) of a row
  // are 16 contiguous, 4-byte aligned bytes, loaded once per four stages (a
  // scale load gives every lane a different row, so its cost is per
  // instruction, not per byte).  Groups past G in the last block belong to
  // stages that are never computed.
  uint4 sblk[SROWS];
  auto sbload = [&](int s) {
    if constexpr (MODE != 1 && KG == 2 && SCD) {
#pragma unroll
      for (int r = 0; r < SROWS; ++r) {
        uint4 v = uint4{0u, 0u, 0u, 0u};
        if (s_live[r])  // wave-uniform
          v = __builtin_bit_cast(uint4, s_is_w[r] ? __builtin_amdgcn_raw_buffer_load_b128(wsres, soff[r] + 4 * (s + s_off), 0, 0)
                                                  : __builtin_amdgcn_raw_buffer_load_b128(asres, soff[r] + 4 * (s + s_off), 0, 0));
        sblk[r] = v;
      }
    }
  };
  auto sstore = [&](int buf, auto kdc) {
    constexpr int KD = decltype(kdc)::value;  // this stage's dword of the scale block
    uint8_t* base = sm + buf * STAGE;
#pragma unroll
    for (int r = 0; r < CHUNKS; ++r) {
      const int row = (tid + NT * r) / PARTS;
      uint8_t* dst = base + row * ROWB;
      *(uint4*)(dst + (((2 * part) ^ (row & 7)) << 4)) = nib_lo16(rc[r]);
      *(uint4*)(dst + (((2 * part + 1) ^ (row & 7)) << 4)) = nib_hi16(rc[r]);
    }
    if constexpr (MODE != 1) {
#pragma unroll
      for (int r = 0; r < SROWS; ++r) {
        const int row = tid + NT * r;
        if (s_live[r]) {
          if constexpr (KG == 2 && SCD) {
            const uint32_t v = KD == 0 ? sblk[r].x : KD == 1 ? sblk[r].y : KD == 2 ? sblk[r].z : sblk[r].w;
            ssc[buf * SC_STAGE + row] = uint2{v & 0xFFFFu, 0u};
            ssc[buf * SC_STAGE + NROWS + row] = uint2{v >> 16, 0u};
          } else {
#pragma unroll
            for (int gg = 0; gg < KG; ++gg) ssc[buf * SC_STAGE + gg * NROWS + row] = uint2{rs[r][gg], 0u};
          }
        }
      }
    }
  };

  v4f acc[BI][BJ];
#pragma unroll
  for (int i = 0; i < BI; ++i)
#pragma unroll
    for (int j = 0; j < BJ; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
  v4i cinit;
#pragma unroll
  for (int v = 0; v < 4; ++v) cinit[v] = MODE != 1 ? kMagicBits : 0;
  const v16f zero16 = {};

  // Pipeline buffers: the 2x2 quads of 16x16 blocks alternate between two
  // sets of (four group products 256*P + c0 bits, one 4-block scale product).
  constexpr int NQ = BI * BJ / 4;
  static_assert(NQ % 2 == 0, "quads alternate between two buffer sets");
  v4i dbuf[2][4];
  v16f sbuf[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
#pragma unroll
    for (int q = 0; q < 4; ++q) dbuf[h][q] = v4i{0, 0, 0, 0};
    sbuf[h] = zero16;
  }

  gload(0);
  sbload(0);
  sstore(0, std::integral_constant<int, 0>{});
  __syncthreads();

  // stage s = 4q + K4 (the phase selects the scale block's dword statically)
  auto stage = [&](int s, auto kc) __attribute__((always_inline)) {
    constexpr int K4 = decltype(kc)::value;
    const int buf = K4 & 1;
    if (s + 1 < lstages) {
      gload(s + 1);
      if constexpr (K4 == 3) sbload(s + 1);
    }
    const uint8_t* base = sm + buf * STAGE;
    // Wave priority: low while multiplying, high while expanding the next
    // stage into LDS and meeting the barrier, so that a wave whose partner
    // on the SIMD (another workgroup) is multiplying gets through its
    // staging first (1.2-2.7% on every shape against either fixed priority
    // or high priority for the multiplications).
    __builtin_amdgcn_s_setprio(0);
#pragma unroll 1
    for (int gg = 0; gg < KG; ++gg) {
      const int g = (s + s_off) * KG + gg;
      // operand fragments of v_mfma_i32_16x16x64_i8: lane = (row l16 of the
      // block, channels 16*lg .. +16 of the group)
      v4i a[BI], b[BJ];
#pragma unroll
      for (int i = 0; i < BI; ++i)
        a[i] = *(const v4i*)(base + (wn + 16 * i + l16) * ROWB + (((4 * gg + lg) ^ (l16 & 7)) << 4));
#pragma unroll
      for (int j = 0; j < BJ; ++j)
        b[j] = *(const v4i*)(base + (BN + wm + 16 * j + l16) * ROWB + (((4 * gg + lg) ^ (l16 & 7)) << 4));
      if constexpr (MODE == 1) {
#pragma unroll
        for (int i = 0; i < BI; ++i)
#pragma unroll
          for (int j = 0; j < BJ; ++j) {
            const v4i d = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[i], b[j], cinit, 0, 0, 0);
            const int m = m0 + wm + 16 * j + l16;
            if (m < M && g < G && n0 + wn < N) {
#pragma unroll
              for (int v = 0; v < 4; ++v) {
                const int n = n0 + wn + 16 * i + 4 * lg + v;
                psums[((size_t)m * N + n) * G + g] = d[v] >> 8;
              }
            }
          }
      } else {
        // Quads Q = (qi, qj) of 2x2 blocks: lane group b of the 4-block scale
        // product v_mfma_f32_16x16x4_4b_f16 is block (2qi + b/2, 2qj + b%2), so
        // this lane supplies the weight scale of row l16 of block row 2qi + lg/2
        // and the activation scale of column l16 of block column 2qj + lg%2.
        // Step Q issues the quad's five matrix instructions and retires quad
        // Q-1 (16 FMAs, independent of what was just issued); the last quad of
        // a group retires at the first step of the next group (the buffers
        // start at zero, so the first retire adds 0 * 0).
        // (the staged 8 bytes are the operands as they stand: no conversion,
        // packing or register moves in the loop; staging fp32 and converting
        // back here cost 8 vector instructions per group and wave)
        const uint2* sc = ssc + buf * SC_STAGE + gg * NROWS;
        uint2 swq[BI / 2], saq[BJ / 2];
#pragma unroll
        for (int qi = 0; qi < BI / 2; ++qi) swq[qi] = sc[wn + 16 * (2 * qi + (lg >> 1)) + l16];
#pragma unroll
        for (int qj = 0; qj < BJ / 2; ++qj) saq[qj] = sc[BN + wm + 16 * (2 * qj + (lg & 1)) + l16];
#pragma unroll
        for (int Q = 0; Q < NQ; ++Q) {
          const int qi = Q / (BJ / 2), qj = Q % (BJ / 2);
          {  // (scale, 0, 0, 0): k = 0 of the lane's block
            const v4h aw4 = __builtin_bit_cast(v4h, swq[qi]);
            const v4h bx4 = __builtin_bit_cast(v4h, saq[qj]);
            sbuf[Q & 1] = __builtin_amdgcn_mfma_f32_16x16x4f16(aw4, bx4, zero16, 0, 0, 0);
          }
#pragma unroll
          for (int q = 0; q < 4; ++q)
            dbuf[Q & 1][q] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[2 * qi + (q >> 1)], b[2 * qj + (q & 1)], cinit, 0, 0, 0);
          const int Qp = Q == 0 ? NQ - 1 : Q - 1;
          const int pi = Qp / (BJ / 2), pj = Qp % (BJ / 2);
#pragma unroll
          for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int v = 0; v < 4; ++v)
              acc[2 * pi + (q >> 1)][2 * pj + (q & 1)][v] =
                  fmaf(sbuf[Qp & 1][4 * q + v], __int_as_float(dbuf[Qp & 1][q][v]),
                       acc[2 * pi + (q >> 1)][2 * pj + (q & 1)][v]);
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
    __builtin_amdgcn_s_setprio(1);
    if (s + 1 < lstages) sstore(buf ^ 1, std::integral_constant<int, (K4 + 1) & 3>{});
    __syncthreads();
  };
  {
    int s = 0;
    for (; s + 3 < lstages; s += 4) {
      stage(s, std::integral_constant<int, 0>{});
      stage(s + 1, std::integral_constant<int, 1>{});
      stage(s + 2, std::integral_constant<int, 2>{});
      stage(s + 3, std::integral_constant<int, 3>{});
    }
    if (s < lstages) stage(s, std::integral_constant<int, 0>{});
    if (s + 1 < lstages) stage(s + 1, std::integral_constant<int, 1>{});
    if (s + 2 < lstages) stage(s + 2, std::integral_constant<int, 2>{});
  }

  if constexpr (MODE != 1) {
    {  // retire the last quad of the last group
      constexpr int Qp = NQ - 1;
      constexpr int pi = Qp / (BJ / 2), pj = Qp % (BJ / 2);
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int v = 0; v < 4; ++v)
          acc[2 * pi + (q >> 1)][2 * pj + (q & 1)][v] =
              fmaf(sbuf[Qp & 1][4 * q + v], __int_as_float(dbuf[Qp & 1][q][v]),
                   acc[2 * pi + (q >> 1)][2 * pj + (q & 1)][v]);
    }
    if constexpr (kTailSplit) {
      // a K slice: partials through the workspace; the tile's last slice
      // continues with the sum of all of them
      if (slice >= 0 &&
          !split_exchange<BI * BJ>(ts, tail_idx, slice, wave, lane, tid, (unsigned*)sm,
                                   [&](int k) { return acc[k / BJ][k % BJ]; },
                                   [&](int k, v4f v) { acc[k / BJ][k % BJ] = v; }))
        return;
    }
    if constexpr (SPLIT == 2) {
      // the second copy's accumulators, through its own staging LDS (every
      // wave passed the loop's last barrier, so that space is free; the
      // epilogue below uses only the first copy's)
      v4f* xch = (v4f*)(smem + LDS_BYTES) + wave * (BI * BJ * 64) + lane;
      if (half == 1) {
#pragma unroll
        for (int i = 0; i < BI; ++i)
#pragma unroll
          for (int j = 0; j < BJ; ++j) xch[(i * BJ + j) * 64] = acc[i][j];
      }
      __syncthreads();
      if (half == 1) return;
#pragma unroll
      for (int i = 0; i < BI; ++i)
#pragma unroll
        for (int j = 0; j < BJ; ++j) {
          const v4f o = xch[(i * BJ + j) * 64];
#pragma unroll
          for (int v = 0; v < 4; ++v) acc[i][j][v] += o[v];
        }
    }
    // Epilogue.  Every global load it needs (bias, the scale rows of the
    // sum_g S product, the first low-rank slices) is issued before any of them
    // is consumed, so the workgroup pays one memory latency here, not several.
    // (branch-free buffer loads: rows past N or M, groups past G and rank
    // slices past r read as zero)
    constexpr int kOutE = 0x7FFFFFF0;
    const __amdgpu_buffer_rsrc_t bres = __builtin_amdgcn_make_buffer_rsrc((void*)bias, (short)0, bias ? N * 2 : 0, kBufDword3);
    const __amdgpu_buffer_rsrc_t l2res = __builtin_amdgcn_make_buffer_rsrc((void*)l2t, (short)0, N * rank * 2, kBufDword3);
    const __amdgpu_buffer_rsrc_t x1res = __builtin_amdgcn_make_buffer_rsrc((void*)xl1, (short)0, M * rank * 4, kBufDword3);
    uint2 bb[BI];
#pragma unroll
    for (int i = 0; i < BI; ++i) {
      const int n = n0 + wn + 16 * i + 4 * lg;
      bb[i] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(bres, n * 2, 0, 0));
    }
    // Inputs of the attention-projection epilogue (MODE 2), issued early so
    // that their latency overlaps the scale-sum and low-rank products: the
    // norm weights of this lane's columns here, the rotary (cos, sin) pairs of
    // its tokens once the scale-sum operands are dead (register budget of two
    // workgroups per CU).  The part (Q, K or V) is the same for the whole
    // workgroup, as heads * head_dim is a multiple of the 128-column tile.
    const int qpart = MODE == 2 ? qkv_part(n0 + wn, qe) : 2;
    const int qc0 = MODE == 2 ? qkv_channel(n0 + wn, qe) : 0;  // 0, or 64 in a 128-channel head's second half
    uint2 wv[BI];
    float4 cs[BI][BJ];
    if (MODE == 2 && qpart < 2) {
      const uint16_t* wnorm = qpart == 0 ? qe.norm_q : qe.norm_k;
#pragma unroll
      for (int i = 0; i < BI; ++i) wv[i] = *(const uint2*)(wnorm + qc0 + 16 * i + 4 * lg);
    }
    // 8 fp16 scales of one row from group g0 (zeros past G and past the tensor)
    auto load8h = [&](__amdgpu_buffer_rsrc_t res, int row, int g0) -> v8h {
      if ((G & 7) == 0)  // rows of 8k groups: one 16-byte load
        return __builtin_bit_cast(v8h, __builtin_amdgcn_raw_buffer_load_b128(res, g0 < G ? (row * G + g0) * 2 : kOutE, 0, 0));
      u32 w[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const u32 lo = __builtin_amdgcn_raw_buffer_load_b16(res, g0 + 2 * e < G ? (row * G + g0 + 2 * e) * 2 : kOutE, 0, 0);
        const u32 hi = __builtin_amdgcn_raw_buffer_load_b16(res, g0 + 2 * e + 1 < G ? (row * G + g0 + 2 * e + 1) * 2 : kOutE, 0, 0);
        w[e] = lo | (hi << 16);
      }
      return __builtin_bit_cast(v8h, uint4{w[0], w[1], w[2], w[3]});
    };
    v8h aw[2][BI], bx[2][BJ];
    auto load_ts = [&](int kb, int h) {
#pragma unroll
      for (int i = 0; i < BI; ++i) aw[h][i] = load8h(wsres, n0 + wn + 16 * i + l16, kb + 8 * lg);
#pragma unroll
      for (int j = 0; j < BJ; ++j) bx[h][j] = load8h(asres, m0 + wm + 16 * j + l16, kb + 8 * lg);
    };
    v8bf al[BI];
    float4 xf[2 * BJ];
    auto load_lr = [&](int jb) {
      const bool live = jb + 8 * lg < rank;  // rank 16 leaves lane groups 2, 3 empty
#pragma unroll
      for (int i = 0; i < BI; ++i) {
        const int n = n0 + wn + 16 * i + l16;
        al[i] = __builtin_bit_cast(v8bf, __builtin_amdgcn_raw_buffer_load_b128(
                                             l2res, live ? (n * rank + jb + 8 * lg) * 2 : kOutE, 0, 0));
      }
#pragma unroll
      for (int j = 0; j < BJ; ++j) {
        const int m = m0 + wm + 16 * j + l16;
        const int off = live ? (m * rank + jb + 8 * lg) * 4 : kOutE;
        xf[2 * j] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(x1res, off, 0, 0));
        xf[2 * j + 1] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(x1res, live ? off + 16 : kOutE, 0, 0));
      }
    };
    load_ts(0, 0);
    if (G > 32) load_ts(32, 1);
    if (rank > 0) load_lr(0);

    // y = 2^18 (acc - c0 sum_g S), formed as (acc (-1/c0) + sum_g S) (-c0 2^18):
    // the matrix core adds sum_g S = Sw . Sa^T (v_mfma_f32_16x16x32_f16, K = 32
    // groups per instruction, exact fp16 products) into the accumulators
    // themselves, so no vector instruction per group of 32 remains.  The one
    // extra rounding, of acc (-1/c0), is 2^-24 of the offset c0 sum_g S.
    const float c0 = __int_as_float(kMagicBits);
    const float neg_inv_c0 = -1.0f / c0;
#pragma unroll
    for (int i = 0; i < BI; ++i)
#pragma unroll
      for (int j = 0; j < BJ; ++j)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[i][j][v] *= neg_inv_c0;
    for (int kb = 0; kb < G; kb += 64) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        if (kb + 32 * h >= G) break;
#pragma unroll
        for (int i = 0; i < BI; ++i)
#pragma unroll
          for (int j = 0; j < BJ; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(aw[h][i], bx[h][j], acc[i][j], 0, 0, 0);
      }
      if (kb + 64 < G) load_ts(kb + 64, 0);
      if (kb + 96 < G) load_ts(kb + 96, 1);
    }
    if (MODE == 2 && qpart < 2) {
      int row[BJ];
      rope_rows_of<BJ, 16>(m0 + wm + l16, qe, row);
#pragma unroll
      for (int j = 0; j < BJ; ++j)
#pragma unroll
        for (int i = 0; i < BI; ++i)
          cs[i][j] = qe.rope ? *(const float4*)(qe.rope + (size_t)row[j] * qe.head_dim + qc0 + 16 * i + 4 * lg)
                             : float4{1.0f, 0.0f, 1.0f, 0.0f};
    }
    const float out_scale = -c0 * kMagicScale;  // exact: c0 times a power of two
#pragma unroll
    for (int i = 0; i < BI; ++i)
#pragma unroll
      for (int j = 0; j < BJ; ++j)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[i][j][v] *= out_scale;

    // low-rank up-projection on the bf16 matrix cores (v_mfma_f32_16x16x32_bf16):
    // acc += L2^T[n, :] . XL1[m, :]; lane = (row l16, rank entries 8*lg .. +8)
    for (int jb = 0; jb < rank; jb += 32) {
      if (jb > 0) load_lr(jb);
      v8bf bl[BJ];
#pragma unroll
      for (int j = 0; j < BJ; ++j) {
        const float4 f0 = xf[2 * j], f1 = xf[2 * j + 1];
        uint4 pk;
        pk.x = pack_bf16x2(f0.x, f0.y);
        pk.y = pack_bf16x2(f0.z, f0.w);
        pk.z = pack_bf16x2(f1.x, f1.y);
        pk.w = pack_bf16x2(f1.z, f1.w);
        bl[j] = __builtin_bit_cast(v8bf, pk);
      }
#pragma unroll
      for (int i = 0; i < BI; ++i)
#pragma unroll
        for (int j = 0; j < BJ; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al[i], bl[j], acc[i][j], 0, 0, 0);
    }

    constexpr int TROW = BI * 16 * 2 + 16;  // bytes per LDS row of a wave's output tile (+ pad)
    if constexpr (MODE == 2) {
      // Fused attention projection.  The bias joins the projection before the
      // norm; then every Q and K head is normalized per token and rotated, V
      // passes.  This lane holds columns 16i + 4lg .. +3 of the wave's 64 for
      // tokens 16j + l16, so rotary pairs stay in the lane.
      static_assert(WAVES_N == 2 && BI * 16 == 64, "a 128-channel head spans the two column waves");
#pragma unroll
      for (int i = 0; i < BI; ++i) {
        const float b[4] = {bf16_bits_to_f32(bb[i].x & 0xFFFFu), bf16_bits_to_f32(bb[i].x >> 16),
                            bf16_bits_to_f32(bb[i].y & 0xFFFFu), bf16_bits_to_f32(bb[i].y >> 16)};
#pragma unroll
        for (int j = 0; j < BJ; ++j)
#pragma unroll
          for (int v = 0; v < 4; ++v) acc[i][j][v] += b[v];
      }
      if (qpart < 2) {
        float ss[BJ];
#pragma unroll
        for (int j = 0; j < BJ; ++j) {
          float t = 0.0f;
#pragma unroll
          for (int i = 0; i < BI; ++i)
#pragma unroll
            for (int v = 0; v < 4; ++v) t = fmaf(acc[i][j][v], acc[i][j][v], t);
          ss[j] = sum_over_rows16(t);  // the wave's 64 columns
        }
        if (qe.head_dim == 128) {  // the head's other 64 columns are the partner wave's (wn ^ 64)
          float* red = (float*)(smem + (NT / 64) * (BJ * 16) * TROW);  // past the output tiles
          if (lg == 0) {
#pragma unroll
            for (int j = 0; j < BJ; ++j) red[wave * 64 + 16 * j + l16] = ss[j];
          }
          __syncthreads();
#pragma unroll
          for (int j = 0; j < BJ; ++j) ss[j] += red[(wave ^ WAVES_M) * 64 + 16 * j + l16];
        }
#pragma unroll
        for (int j = 0; j < BJ; ++j) {
          const float r = inv_rms(ss[j], qe);
#pragma unroll
          for (int i = 0; i < BI; ++i) {
            const float4 o = norm_rope4(acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3], r, wv[i], cs[i][j]);
            acc[i][j] = v4f{o.x, o.y, o.z, o.w};
          }
        }
      }
    }

    if constexpr (MODE == 3) {
#pragma clang fp contract(off)
      // Fused MLP up-projection.  y (+ bias) -> h = bf16(GELU(y)), then the
      // down projection's activation quantization of h, exactly as
      // svdq_quantize_act would do on a bf16 input: xh = fl32(h * fl32(1/lambda)),
      // s = fp16_sat(fl32(amax / 7)) over the 64 channels of a group (this
      // wave's 64 columns), q = clamp(rne(fl32(xh * fl32(1/s))), -8, 7); and
      // the low-rank input XL1 += h . L1 over this wave's columns (fp32
      // atomics: every column tile adds its share).  Y is never written.
      const int nw = n0 + wn;  // first column of this wave: the first channel of its group
      const int G2 = N >> 6, gd = nw >> 6;
      u32 hp[BI][BJ][2];       // h as bf16 pairs (channels 4lg + {0,1}, {2,3} of block i)
      float rl[BI][4];
#pragma unroll
      for (int i = 0; i < BI; ++i) {
        const float b[4] = {bf16_bits_to_f32(bb[i].x & 0xFFFFu), bf16_bits_to_f32(bb[i].x >> 16),
                            bf16_bits_to_f32(bb[i].y & 0xFFFFu), bf16_bits_to_f32(bb[i].y >> 16)};
        const uint2 lw = me.lam ? *(const uint2*)(me.lam + nw + 16 * i + 4 * lg) : uint2{0x3F803F80u, 0x3F803F80u};
        rl[i][0] = 1.0f / bf16_bits_to_f32(lw.x & 0xFFFFu);
        rl[i][1] = 1.0f / bf16_bits_to_f32(lw.x >> 16);
        rl[i][2] = 1.0f / bf16_bits_to_f32(lw.y & 0xFFFFu);
        rl[i][3] = 1.0f / bf16_bits_to_f32(lw.y >> 16);
#pragma unroll
        for (int j = 0; j < BJ; ++j) {
          float h[4];
#pragma unroll
          for (int v = 0; v < 4; ++v) h[v] = gelu_f32(acc[i][j][v] + b[v]);
          hp[i][j][0] = pack_bf16x2(h[0], h[1]);
          hp[i][j][1] = pack_bf16x2(h[2], h[3]);
          acc[i][j][0] = bf16_bits_to_f32(hp[i][j][0] & 0xFFFFu) * rl[i][0];  // xh
          acc[i][j][1] = bf16_bits_to_f32(hp[i][j][0] >> 16) * rl[i][1];
          acc[i][j][2] = bf16_bits_to_f32(hp[i][j][1] & 0xFFFFu) * rl[i][2];
          acc[i][j][3] = bf16_bits_to_f32(hp[i][j][1] >> 16) * rl[i][3];
        }
      }
      // codes through LDS (free after the main loop): this wave's 64 tokens x
      // 32 bytes; lane writes 2 bytes per block, then 16-byte row stores
      constexpr int CROW = 48;  // bytes per LDS row (32 + pad)
      uint8_t* ct = smem + wave * (BJ * 16) * CROW;
#pragma unroll
      for (int j = 0; j < BJ; ++j) {
        float a = 0.0f;
#pragma unroll
        for (int i = 0; i < BI; ++i)
#pragma unroll
          for (int v = 0; v < 4; ++v) a = fmaxf(a, fabsf(acc[i][j][v]));
        a = max_over_rows16(a);
        const u32 sbits = f32_to_f16_sat_bits(a / 7.0f);
        const float sf = f16_bits_to_f32(sbits);
        const float t = sf == 0.0f ? 0.0f : 1.0f / sf;
#pragma unroll
        for (int i = 0; i < BI; ++i) {
          u32 w = 0u;
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            float q = __builtin_rintf(acc[i][j][v] * t);
            q = fminf(fmaxf(q, -8.0f), 7.0f);
            w |= ((u32)(int)q & 0xFu) << (4 * v);
          }
          *(uint16_t*)(ct + (16 * j + l16) * CROW + 8 * i + 2 * lg) = (uint16_t)w;
        }
        const int m = m0 + wm + 16 * j + l16;
        if (lg == 0 && m < M) ((uint16_t*)me.scales)[(size_t)m * G2 + gd] = (uint16_t)sbits;
      }
#pragma unroll
      for (int rr = 0; rr < BJ * 16 * 2 / 64; ++rr) {  // 64 rows x 2 halves, 64 lanes per pass
        const int row = rr * 32 + (lane >> 1), half = lane & 1;
        const uint4 v = *(const uint4*)(ct + row * CROW + 16 * half);
        const int m = m0 + wm + row;
        if (m < M) *(uint4*)(me.codes + (size_t)m * (N >> 1) + gd * 32 + 16 * half) = v;
      }
      // XL1 += h . L1 on the bf16 matrix cores (v_mfma_f32_16x16x32_bf16):
      // A = h [tokens x 32 channels] with this lane's own channels as its k
      // slots (16*(2c) + 4lg + 0..3, then 16*(2c+1) + 4lg + 0..3), B = L1 with
      // the same channel order; D[4lg + v][l16] = token 16j + 4lg + v, rank
      // column rb*16 + l16.  The two column waves of a row block cover the
      // same tokens: the second puts its partial in LDS, the first adds it to
      // its own (a fixed order) and makes the one atomic add per element.  The
      // exchange space alternates between two halves from one 16-rank block
      // to the next, so one barrier per block keeps writes clear of reads.
      static_assert(WAVES_N == 2, "column waves pair up for the XL1 exchange");
      const int cw = wave / WAVES_M, rw = wave % WAVES_M;
      float* const xx = (float*)(smem + (NT / 64) * (BJ * 16) * CROW);  // [2][WAVES_M][BJ*4][64]
      static_assert((NT / 64) * (BJ * 16) * CROW + 2 * WAVES_M * BJ * 4 * 64 * 4 <= LDS_BYTES,
                    "codes tiles and the XL1 exchange fit the staging LDS");
      int par = 0;
      for (int rb = 0; rb < me.rank; rb += 16, par ^= 1) {
        const int r = rb + l16;
        v8bf bl[2];
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const uint2 lo = *(const uint2*)(me.l1t + (size_t)r * N + nw + 32 * c + 4 * lg);
          const uint2 hi = *(const uint2*)(me.l1t + (size_t)r * N + nw + 32 * c + 16 + 4 * lg);
          bl[c] = __builtin_bit_cast(v8bf, uint4{lo.x, lo.y, hi.x, hi.y});
        }
        v4f d[BJ];
#pragma unroll
        for (int j = 0; j < BJ; ++j) {
          d[j] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int c = 0; c < 2; ++c) {
            const v8bf al = __builtin_bit_cast(
                v8bf, uint4{hp[2 * c][j][0], hp[2 * c][j][1], hp[2 * c + 1][j][0], hp[2 * c + 1][j][1]});
            d[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bl[c], d[j], 0, 0, 0);
          }
        }
        float* const xp = xx + (par * WAVES_M + rw) * (BJ * 4 * 64) + lane;
        if (cw == 1) {
#pragma unroll
          for (int j = 0; j < BJ; ++j)
#pragma unroll
            for (int v = 0; v < 4; ++v) xp[(4 * j + v) * 64] = d[j][v];
        }
        __syncthreads();
        if (cw == 0) {
#pragma unroll
          for (int j = 0; j < BJ; ++j)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
              const int m = m0 + wm + 16 * j + 4 * lg + v;
              if (m < M) unsafeAtomicAdd(me.xl1 + (size_t)m * me.rank + r, d[j][v] + xp[(4 * j + v) * 64]);
            }
        }
      }
      return;
    }

    // bias (MODE 0), bf16 rounding, then the wave's tile goes through LDS
    // (free after the main loop) so that each store instruction writes whole
    // 128-byte row segments of Y: lane l of a store covers row l/8, bytes
    // 16*(l%8) .. +16.
    static_assert((NT / 64) * (BJ * 16) * TROW + NT * 4 <= LDS_BYTES, "output tiles and norm sums fit in LDS");
    uint8_t* tile = smem + wave * (BJ * 16) * TROW;
#pragma unroll
    for (int i = 0; i < BI; ++i) {
      const float b0 = bf16_bits_to_f32(bb[i].x & 0xFFFFu), b1 = bf16_bits_to_f32(bb[i].x >> 16);
      const float b2 = bf16_bits_to_f32(bb[i].y & 0xFFFFu), b3 = bf16_bits_to_f32(bb[i].y >> 16);
#pragma unroll
      for (int j = 0; j < BJ; ++j) {
        uint2 o;
        if constexpr (MODE == 2) {  // bias already in
          o.x = pack_bf16x2(acc[i][j][0], acc[i][j][1]);
          o.y = pack_bf16x2(acc[i][j][2], acc[i][j][3]);
        } else {
          o.x = pack_bf16x2(acc[i][j][0] + b0, acc[i][j][1] + b1);
          o.y = pack_bf16x2(acc[i][j][2] + b2, acc[i][j][3] + b3);
        }
        *(uint2*)(tile + (16 * j + l16) * TROW + (16 * i + 4 * lg) * 2) = o;
      }
    }
    if (n0 + wn < N) {
      constexpr int LPR = BI * 16 * 2 / 16;  // lanes per tile row (16 bytes each)
      constexpr int RPI = 64 / LPR;          // tile rows per store instruction
#pragma unroll
      for (int r0 = 0; r0 < BJ * 16; r0 += RPI) {
        const int r = r0 + lane / LPR, c = lane % LPR;
        const uint4 v = *(const uint4*)(tile + r * TROW + c * 16);
        const int m = m0 + wm + r;
        if (m < M) *(uint4*)(y + (size_t)m * N + n0 + wn + c * 8) = v;
      }
    }
  }
}

// The plain grid's last partial round, split along K when a workspace is
// given: grids of more than one round of two tiles per CU whose last round
// holds at most an eighth of a round (2592 tiles of the 4608 x 9216 QKV shape:
// 32 left on 512 slots), with at least eight two-group stages.  Measured on
// that shape: 2, 3, 4 and 6 slices per tile all take ~200 us against 206.5 us
// unsplit; 8 slices 205.7 us.
static TailSplit tail_split(int blocks, int groups, void* work) {
  TailSplit ts{};
  const int slots = 2 * device_cu_count(), stages = (groups + KG - 1) / KG;
  if (!work || (blocks & 7) || (slots & 7) || blocks <= slots || stages < 8) return ts;
  const int tail = blocks % slots;  // a multiple of 8 (blocks and slots are)
  if (tail == 0 || tail > slots / 8 || tail > kTailMaxTiles) return ts;
  ts.full = blocks - tail;
  ts.tail = tail;
  ts.parts = kTailParts;
  ts.part = (float*)work;
  ts.cnt = (unsigned*)((uint8_t*)work + kTailPartBytes);
  return ts;
}

// Test hook: when set, the plain GEMM never takes the K-split instance.
static std::atomic<int> g_no_ksplit{0};
void set_no_ksplit(int v) { g_no_ksplit.store(v ? 1 : 0); }

hipError_t launch_gemm_int4(const GemmArgs& a, hipStream_t st) {
  const int m_tiles = (int)((a.M + BM - 1) / BM);
  const int blocks = m_tiles * (int)((a.N + BN - 1) / BN);
  // an even group count makes a row's scales of four stages one 16-byte block
  const bool scd = (a.K / 64) % 2 == 0;
  auto k0 = scd ? gemm_int4_kernel<0, true, 1> : gemm_int4_kernel<0, false, 1>;
  auto k1 = gemm_int4_kernel<1, false, 1>;
  auto k2 = scd ? gemm_int4_kernel<2, true, 1> : gemm_int4_kernel<2, false, 1>;
  auto k3 = scd ? gemm_int4_kernel<3, true, 1> : gemm_int4_kernel<3, false, 1>;
  auto ks = gemm_int4_kernel<0, true, 2>;
  const void* kf = a.psums ? (const void*)k1 : a.qkv ? (const void*)k2 : a.mlp ? (const void*)k3 : (const void*)k0;
  hipError_t e = hipFuncSetAttribute(kf, hipFuncAttributeMaxDynamicSharedMemorySize, (int)LDS_BYTES);
  if (e != hipSuccess) return e;
  const QkvEpi qnone{};
  const MlpEpi mnone{};
  const TailSplit tnone{};
  if (a.psums) {
    hipLaunchKernelGGL(k1, dim3(blocks), dim3(NT), LDS_BYTES, st, (int)a.M, (int)a.N, (int)a.K, 0,
                       (const uint8_t*)a.act_codes, nullptr, (const uint8_t*)a.w_codes, nullptr, nullptr,
                       nullptr, nullptr, nullptr, (int32_t*)a.psums, qnone, mnone, tnone);
  } else if (a.qkv) {
    const TailSplit ts = tail_split(blocks, (int)(a.K / 64), a.work);
    const int grid = ts.parts > 0 ? ts.full + ts.tail * ts.parts : blocks;
    hipLaunchKernelGGL(k2, dim3(grid), dim3(NT), LDS_BYTES, st, (int)a.M, (int)a.N, (int)a.K, a.rank,
                       (const uint8_t*)a.act_codes, (const uint16_t*)a.act_scales,
                       (const uint8_t*)a.w_codes, (const uint16_t*)a.w_scales, a.xl1,
                       (const uint16_t*)a.l2t, (const uint16_t*)a.bias, (uint16_t*)a.y, nullptr, *a.qkv, mnone, ts);
  } else if (a.mlp) {
    const int nx = (int)(a.M * a.mlp->rank);
    if (nx > 0) hipLaunchKernelGGL(fill_zero_f32, dim3((nx + 255) / 256), dim3(256), 0, st, a.mlp->xl1, nx);
    hipLaunchKernelGGL(k3, dim3(blocks), dim3(NT), LDS_BYTES, st, (int)a.M, (int)a.N, (int)a.K, a.rank,
                       (const uint8_t*)a.act_codes, (const uint16_t*)a.act_scales,
                       (const uint8_t*)a.w_codes, (const uint16_t*)a.w_scales, a.xl1,
                       (const uint16_t*)a.l2t, (const uint16_t*)a.bias, nullptr, nullptr, qnone, *a.mlp, tnone);
  } else {
    // A grid of at most one tile per CU runs on the K-split kernel (needs an
    // even number of two-group stages: K % 256 == 0).  Sending only the last
    // partial round of a larger grid there measured slower: the second launch
    // waits for the whole first grid, which costs more than the lone tiles.
    if ((a.K / 64) % 4 == 0 && blocks <= device_cu_count() && !g_no_ksplit.load()) {
      e = hipFuncSetAttribute((const void*)ks, hipFuncAttributeMaxDynamicSharedMemorySize, (int)(2 * LDS_BYTES));
      if (e != hipSuccess) return e;
      hipLaunchKernelGGL(ks, dim3(blocks), dim3(2 * NT), 2 * LDS_BYTES, st, (int)a.M, (int)a.N, (int)a.K, a.rank,
                         (const uint8_t*)a.act_codes, (const uint16_t*)a.act_scales,
                         (const uint8_t*)a.w_codes, (const uint16_t*)a.w_scales, a.xl1,
                         (const uint16_t*)a.l2t, (const uint16_t*)a.bias, (uint16_t*)a.y, nullptr, qnone, mnone, tnone);
    } else {
      const TailSplit ts = tail_split(blocks, (int)(a.K / 64), a.work);
      const int grid = ts.parts > 0 ? ts.full + ts.tail * ts.parts : blocks;
      hipLaunchKernelGGL(k0, dim3(grid), dim3(NT), LDS_BYTES, st, (int)a.M, (int)a.N, (int)a.K, a.rank,
                         (const uint8_t*)a.act_codes, (const uint16_t*)a.act_scales,
                         (const uint8_t*)a.w_codes, (const uint16_t*)a.w_scales, a.xl1,
                         (const uint16_t*)a.l2t, (const uint16_t*)a.bias, (uint16_t*)a.y, nullptr, qnone, mnone, ts);
    }
  }
  return hipGetLastError();
}

}  // namespace svdq
