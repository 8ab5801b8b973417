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
// the down projection (int4, group 64, smoothing lam or NULL) into codes
// [M, N/2] and fp16 scales [M, N/64], and XL1 = h . L1 [M, rank] is summed
// into xl1 (zeroed by the launcher) from every column tile.
struct MlpEpi {
  const uint16_t* lam;
  const uint16_t* l1t;  // L1^T [rank, N]
  int rank;
  uint8_t* codes;
  uint16_t* scales;
  float* xl1;
};

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
hipError_t launch_lowrank(const LowrankArgs& a, hipStream_t st);
hipError_t launch_quantize_weight(int precision, int64_t N, int64_t K, const float* r, float alpha, void* codes,
                                  void* scales, hipStream_t st);
hipError_t launch_awq_quantize(int64_t N, int64_t K, const void* w, void* codes, void* scales, void* zeros,
                               hipStream_t st);
hipError_t launch_gemm_int4(const GemmArgs& a, hipStream_t st);
hipError_t launch_gemm_nvfp4(const GemmArgs& a, hipStream_t st);
hipError_t launch_awq(const AwqArgs& a, hipStream_t st);

}  // namespace svdq
