// Internal launch interface between the C-ABI layer (svdq_api.hip) and the
// kernel files.  Arguments arrive already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace svdq {

// Compute units of the current device (cached per device).
inline int device_cu_count() {
  static int cus[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cus[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cus[dev] = n;
  }
  return cus[dev];
}

struct QuantArgs {
  int precision, rank;
  int64_t M, K;
  const void* x;
  const void* smooth;
  const void* l1t;
  float alpha;
  void* codes;
  void* scales;
  float* xl1;
  void* work;  // svdq_quantize_act_ws: the GEMM workspace (counters zero), or null
};

// Epilogue of the fused attention projection: columns [Q | K | V], each hd =
// heads * head_dim wide; Q and K heads get RMSNorm (weights norm_q / norm_k,
// epsilon eps) and then the rotary embedding from rope [rope_rows, head_dim/2, 2]
// (cos, sin) pairs, token row m using table row m % rope_rows (rope may be null).
struct QkvEpi {
  int hd, head_dim;
  const uint16_t* norm_q;
  const uint16_t* norm_k;
  float eps;
  const float* rope;
  int rope_rows;
};

// Epilogue of the fused MLP up-projection: h = bf16(GELU(y)) is quantized for
// the down projection (smoothing lam or NULL; the GEMM's precision: int4 group
// 64 with fp16 scales [M, N/64], or nvfp4 group 16 with E4M3 scales [M, N/16]
// and the global scale alpha) into codes [M, N/2], and XL1 = h . L1 [M, rank]
// is summed into xl1 (zeroed by the launcher) from every column tile.
struct MlpEpi {
  const uint16_t* lam;
  const uint16_t* l1t;  // L1^T [rank, N]
  int rank;
  uint8_t* codes;
  void* scales;
  float* xl1;
  float alpha;  // nvfp4: the down projection's activation global scale
};

// The last partial round of the plain int4 GEMM's tile grid, split along K.
// Blocks [0, full) run whole tiles; the tiles left over (tail of them, the
// last tail/8 of each XCD's range of the tile order) run as `parts` K slices
// each, in blocks [full, full + tail * parts) of the same launch.  A slice
// stores its fp32 accumulators in part, counts itself in cnt[tile], and the
// last of a tile's slices to arrive sums all of them in slice order and runs
// the epilogue.  cnt holds zeros between calls (the last slice resets it).
struct TailSplit {
  int full, tail, parts;  // parts == 0: no split
  float* part;            // [tail][parts][NT/64 waves][BI*BJ blocks][2 halves][64 lanes][2]
  unsigned* cnt;          // [tail]
};

// Workspace of the split tail (svdq_w4a4_gemm_ws): partial tiles of up to
// kTailMaxTiles tiles x kTailParts slices, then one counter per tile.
constexpr int kTailMaxTiles = 64, kTailParts = 4;
constexpr size_t kTailTileBytes = (size_t)128 * 128 * 4;  // fp32 accumulators of one 128 x 128 tile
constexpr size_t kTailPartBytes = (size_t)kTailMaxTiles * kTailParts * kTailTileBytes;
constexpr size_t kGemmWorkBytes = kTailPartBytes + 4096;

// The balanced quantizer (svdq_quantize_act_ws): the grid of (32-row block,
// 64-channel step) pairs cut into equal contiguous ranges of L steps, one per
// workgroup, L <= steps per block, so a block is shared by workgroups only at
// range ends.  The XL1 rows of a shared block are summed from the pieces'
// fp32 partial tiles in part (two slots per workgroup) by the last piece to
// arrive, counted in cnt[first workgroup of the block].  Both live in the
// GEMM workspace: part in its partial-tile area (scratch), cnt in its counter
// page above the GEMM's counters, zero between calls like those.
struct QuantSplit {
  int L, T;       // steps per workgroup (0: one block per workgroup), blocks * steps
  float* part;    // [2 * workgroups][32 rows][rank]
  unsigned* cnt;  // [workgroups]
};
constexpr int kQuantMaxGroups = 512;
constexpr size_t kQuantCntOffset = kTailPartBytes + 1024;
static_assert((size_t)kQuantMaxGroups * 2 * 32 * 32 * 4 <= kTailPartBytes, "quantizer partials fit the workspace");
static_assert((size_t)kTailMaxTiles * 4 <= 1024 && 1024 + (size_t)kQuantMaxGroups * 4 <= 4096,
              "GEMM and quantizer counters share the counter page without overlap");

struct GemmArgs {
  int precision, rank;
  int64_t M, N, K;
  const void* act_codes;
  const void* act_scales;
  float alpha_a;
  const void* w_codes;
  const void* w_scales;
  float alpha_w;
  const float* xl1;
  const void* l2t;
  const void* bias;
  void* y;       // bf16 [M, N] (GEMM) ...
  void* psums;   // ... or [M, N, K/G] partial products (test support)
  const QkvEpi* qkv;  // non-null: Y with the Q/K norm and rotary epilogue
  const MlpEpi* mlp;  // non-null: no Y; GELU + the next layer's quantization
  void* work;         // plain int4 GEMM: kGemmWorkBytes, counters zero, or null
};

struct AwqArgs {
  int64_t M, N, K;
  const void* x;
  const void* w_codes;
  const void* w_scales;
  const void* w_zeros;
  const void* bias;
  void* y;
};

struct LowrankArgs {
  int64_t N, K;
  int rank, p, iters;
  const void* w;
  const void* lam;
  const float* omega;
  void* l1t;
  void* l2t;
  float* residual;
  void* work;
};

hipError_t launch_quantize_act(const QuantArgs& a, hipStream_t st);
hipError_t launch_calibrate(int64_t Mc, int64_t N, int64_t K, const void* x, const void* w, void* lam, hipStream_t st);
size_t lowrank_workspace_bytes(int64_t N, int64_t K, int p);
// The allocation-free decomposition's fixed workspace: its size, and its device
// address on the current device (looked up once per device).
constexpr size_t kNoAllocScratchBytes = (size_t)16 << 20;
hipError_t noalloc_scratch(void** ptr);
hipError_t launch_lowrank(const LowrankArgs& a, hipStream_t st);
hipError_t launch_quantize_weight(int precision, int64_t N, int64_t K, const float* r, float alpha, void* codes,
                                  void* scales, hipStream_t st);
hipError_t launch_awq_quantize(int64_t N, int64_t K, const void* w, void* codes, void* scales, void* zeros,
                               hipStream_t st);
hipError_t launch_gemm_int4(const GemmArgs& a, hipStream_t st);
void set_no_ksplit(int v);
hipError_t launch_gemm_nvfp4(const GemmArgs& a, hipStream_t st);
hipError_t launch_awq(const AwqArgs& a, hipStream_t st);
// The quantizer and an independent AWQ GEMV (either may be null): one fused
// launch where both shapes allow it (quant_awq_fusable), else the two
// launches in that order.
bool quant_awq_fusable(const QuantArgs& q, const AwqArgs& w, int* sx);
hipError_t launch_quant_awq(const QuantArgs* q, const AwqArgs* w, hipStream_t st);

}  // namespace svdq
