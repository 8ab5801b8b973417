// C ABI of libsvdq.so (declared in include/svdq.h): argument validation, the
// device architecture check and dispatch to the gfx950 kernels.  Nothing here
// allocates device memory.
//
// The accepted (method, precision, group) triples are the table in "Nunchaku
// Lite", "Supported quantization types": svdq_w4a4 nvfp4 16, svdq_w4a4 int4
// 64, awq_w4a16 int4 64.  A device that is not gfx950 is rejected with an
// error before any launch, never run into wrong results (blog "Nunchaku 4-bit
// inference in Diffusers", "Hardware support": the capability check at load).
#include <float.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <string>

#include "../../include/svdq.h"
#include "launch.h"

namespace {

thread_local std::string g_last_error;
std::mutex g_arch_mu;
std::string g_arch_override;
bool g_has_override = false;
int g_arch_ok[64];  // per device: 0 unknown, 1 gfx950, 2 other

svdq_status fail(svdq_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

svdq_status ok() {
  g_last_error.clear();
  return SVDQ_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

svdq_status check_arch() {
  std::lock_guard<std::mutex> lk(g_arch_mu);
  if (g_has_override) {
    if (g_arch_override.rfind("gfx950", 0) != 0)
      return fail(SVDQ_ERR_UNSUPPORTED, "device architecture %s is not supported (gfx950 required)",
                  g_arch_override.c_str());
    return SVDQ_OK;
  }
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(SVDQ_ERR_DEVICE, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= 64) return fail(SVDQ_ERR_DEVICE, "device index %d out of range", dev);
  if (g_arch_ok[dev] == 0) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return fail(SVDQ_ERR_DEVICE, "hipGetDeviceProperties: %s", hipGetErrorString(e));
    g_arch_ok[dev] = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    if (g_arch_ok[dev] != 1)
      return fail(SVDQ_ERR_UNSUPPORTED, "device architecture %s is not supported (gfx950 required)",
                  prop.gcnArchName);
  }
  if (g_arch_ok[dev] != 1) return fail(SVDQ_ERR_UNSUPPORTED, "device is not gfx950");
  return SVDQ_OK;
}

// Reports a fault left by an earlier launch, before anything new is enqueued.
svdq_status check_sticky() {
  hipError_t e = hipPeekAtLastError();
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return fail(SVDQ_ERR_DEVICE, "earlier HIP error: %s", hipGetErrorString(e));
  }
  return SVDQ_OK;
}

svdq_status launched(hipError_t e) {
  if (e != hipSuccess) return fail(SVDQ_ERR_DEVICE, "kernel launch: %s", hipGetErrorString(e));
  return ok();
}

bool valid_rank(int r) { return r >= 0 && r <= 128 && r % 16 == 0; }

svdq_status check_precision(int precision, int group) {
  if (precision == SVDQ_INT4 && group == 64) return SVDQ_OK;
  if (precision == SVDQ_NVFP4 && group == 16) return SVDQ_OK;
  return fail(SVDQ_ERR_UNSUPPORTED,
              "svdq_w4a4 supports (int4, group 64) and (nvfp4, group 16); got precision %d group %d",
              precision, group);
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || !na || !nb) return false;
  uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

constexpr int64_t kMaxDim = (int64_t)1 << 30;
constexpr int64_t kMax32 = (int64_t)1 << 31;  // 32-bit byte offsets inside the kernels
// Largest channel count: the quantizer's limit, and the largest K at which the
// GEMMs' fp32 accumulation is parity-tested.
constexpr int64_t kMaxK = 32768;

}  // namespace

extern "C" {

int svdq_abi_version(void) { return 1; }

const char* svdq_last_error(void) { return g_last_error.c_str(); }

void svdq_test_set_arch_override(const char* arch) {
  std::lock_guard<std::mutex> lk(g_arch_mu);
  g_has_override = arch != nullptr;
  g_arch_override = arch ? arch : "";
}

void svdq_test_set_no_ksplit(int on) { svdq::set_no_ksplit(on); }

// Validates a quantizer call; launches it, or with `prep` only fills *prep
// (left untouched for an empty call).
static svdq_status quantize_act(int precision, int group_size, int rank, int64_t M, int64_t K, const void* x,
                                const void* smooth, const void* l1t, float act_global_scale, void* act_codes,
                                void* act_scales, float* xl1, void* stream, void* work, int64_t work_bytes,
                                svdq::QuantArgs* prep = nullptr) {
  svdq_status s;
  if ((s = check_precision(precision, group_size)) != SVDQ_OK) return s;
  if (!valid_rank(rank)) return fail(SVDQ_ERR_UNSUPPORTED, "rank %d not in {0, 16, ..., 128}", rank);
  if (M < 0 || K <= 0 || M > kMaxDim || K > kMaxDim) return fail(SVDQ_ERR_INVALID_ARG, "bad shape M=%lld K=%lld", (long long)M, (long long)K);
  if (K % 64 != 0) return fail(SVDQ_ERR_UNSUPPORTED, "K=%lld must be a multiple of 64", (long long)K);
  if (K > kMaxK) return fail(SVDQ_ERR_UNSUPPORTED, "K=%lld above the supported %lld", (long long)K, (long long)kMaxK);
  if (M * K >= ((int64_t)1 << 30)) return fail(SVDQ_ERR_UNSUPPORTED, "M*K above 2^30 - 1 (x must stay below 2 GiB)");
  if (M * rank * 4 >= kMax32) return fail(SVDQ_ERR_UNSUPPORTED, "M*rank*4 must stay below 2^31 bytes");
  if (M == 0) return ok();  // empty call: nothing to read or write
  if (!x || !act_codes || !act_scales) return fail(SVDQ_ERR_INVALID_ARG, "x, act_codes and act_scales are required");
  if ((rank > 0) != (l1t != nullptr)) return fail(SVDQ_ERR_INVALID_ARG, "l1t must be given iff rank > 0");
  if ((rank > 0) != (xl1 != nullptr)) return fail(SVDQ_ERR_INVALID_ARG, "xl1 must be given iff rank > 0");
  if (precision == SVDQ_NVFP4 && !(act_global_scale > 0.0f && act_global_scale < 3.0e38f))
    return fail(SVDQ_ERR_INVALID_ARG, "act_global_scale must be finite and > 0 for nvfp4");
  if (!aligned16(x) || !aligned16(smooth) || !aligned16(l1t) || !aligned16(act_codes) ||
      !aligned16(act_scales) || !aligned16(xl1))
    return fail(SVDQ_ERR_ALIGNMENT, "all buffers must be 16-byte aligned");
  const size_t nx = (size_t)M * K * 2, nc = (size_t)M * K / 2;
  const size_t ns = precision == SVDQ_INT4 ? (size_t)M * (K / 64) * 2 : (size_t)M * (K / 16);
  const size_t nl = (size_t)M * rank * 4;
  if (overlaps(x, nx, act_codes, nc) || overlaps(x, nx, act_scales, ns) || overlaps(x, nx, xl1, nl) ||
      overlaps(act_codes, nc, act_scales, ns) || overlaps(act_codes, nc, xl1, nl) ||
      overlaps(act_scales, ns, xl1, nl))
    return fail(SVDQ_ERR_INVALID_ARG, "outputs must not overlap each other or x");
  if (work) {
    if (work_bytes < (int64_t)SVDQ_GEMM_WORK_BYTES)
      return fail(SVDQ_ERR_INVALID_ARG, "work_bytes=%lld below SVDQ_GEMM_WORK_BYTES=%lld", (long long)work_bytes,
                  (long long)SVDQ_GEMM_WORK_BYTES);
    if (!aligned16(work)) return fail(SVDQ_ERR_ALIGNMENT, "all buffers must be 16-byte aligned");
    const size_t nw = (size_t)SVDQ_GEMM_WORK_BYTES;
    if (overlaps(work, nw, x, nx) || overlaps(work, nw, act_codes, nc) || overlaps(work, nw, act_scales, ns) ||
        overlaps(work, nw, xl1, nl) || overlaps(work, nw, smooth, (size_t)K * 2) ||
        overlaps(work, nw, l1t, (size_t)rank * K * 2))
      return fail(SVDQ_ERR_INVALID_ARG, "work must not overlap x, an input or an output");
  } else if (work_bytes != 0) {
    return fail(SVDQ_ERR_INVALID_ARG, "work_bytes=%lld given without work", (long long)work_bytes);
  }
  svdq::QuantArgs a{precision, rank, M, K, x, smooth, l1t, act_global_scale, act_codes, act_scales, xl1, work};
  if (prep) {  // the caller checks the device once for both of its jobs
    *prep = a;
    return ok();
  }
  if ((s = check_arch()) != SVDQ_OK) return s;
  if ((s = check_sticky()) != SVDQ_OK) return s;
  return launched(svdq::launch_quantize_act(a, (hipStream_t)stream));
}

svdq_status svdq_quantize_act(int precision, int group_size, int rank, int64_t M, int64_t K,
                              const void* x, const void* smooth, const void* l1t,
                              float act_global_scale, void* act_codes, void* act_scales,
                              float* xl1, void* stream) {
  return quantize_act(precision, group_size, rank, M, K, x, smooth, l1t, act_global_scale, act_codes, act_scales,
                      xl1, stream, nullptr, 0);
}

svdq_status svdq_quantize_act_ws(int precision, int group_size, int rank, int64_t M, int64_t K,
                                 const void* x, const void* smooth, const void* l1t,
                                 float act_global_scale, void* act_codes, void* act_scales,
                                 float* xl1, void* work, int64_t work_bytes, void* stream) {
  return quantize_act(precision, group_size, rank, M, K, x, smooth, l1t, act_global_scale, act_codes, act_scales,
                      xl1, stream, work, work_bytes);
}

static svdq_status gemm_common(int precision, int group_size, int rank, int64_t M, int64_t N,
                               int64_t K, const void* act_codes, const void* w_codes) {
  svdq_status s;
  if ((s = check_precision(precision, group_size)) != SVDQ_OK) return s;
  if (!valid_rank(rank)) return fail(SVDQ_ERR_UNSUPPORTED, "rank %d not in {0, 16, ..., 128}", rank);
  if (M < 0 || N <= 0 || K <= 0 || M > kMaxDim || N > kMaxDim || K > kMaxDim)
    return fail(SVDQ_ERR_INVALID_ARG, "bad shape M=%lld N=%lld K=%lld", (long long)M, (long long)N, (long long)K);
  if (K % 64 != 0) return fail(SVDQ_ERR_UNSUPPORTED, "K=%lld must be a multiple of 64", (long long)K);
  if (K > kMaxK) return fail(SVDQ_ERR_UNSUPPORTED, "K=%lld above the supported %lld", (long long)K, (long long)kMaxK);
  if (N % 128 != 0) return fail(SVDQ_ERR_UNSUPPORTED, "N=%lld must be a multiple of 128", (long long)N);
  if (M * K > ((int64_t)1 << 31) || N * K > ((int64_t)1 << 31) || M * N > ((int64_t)1 << 31))
    return fail(SVDQ_ERR_UNSUPPORTED, "operand above 2^31 elements");
  // the kernels address xl1 [M, rank] fp32 and l2t [N, rank] bf16 with 32-bit byte offsets
  if (M * rank * 4 >= kMax32 || N * rank * 2 >= kMax32)
    return fail(SVDQ_ERR_UNSUPPORTED, "M*rank*4 and N*rank*2 must stay below 2^31 bytes");
  if (M > 0 && !act_codes) return fail(SVDQ_ERR_INVALID_ARG, "act_codes is required");
  if (!w_codes) return fail(SVDQ_ERR_INVALID_ARG, "w_codes is required");
  return SVDQ_OK;
}

// Checks shared by the two Y-producing GEMM entry points; qkv (may be NULL)
// is the attention-projection epilogue.
static svdq_status gemm_y(int precision, int group_size, int rank, int64_t M, int64_t N,
                          int64_t K, const void* act_codes, const void* act_scales,
                          float act_global_scale, const void* w_codes, const void* w_scales,
                          float w_global_scale, const float* xl1, const void* l2t,
                          const void* bias, void* y, void* stream, const svdq::QkvEpi* qkv,
                          size_t rope_bytes, void* work = nullptr) {
  svdq_status s;
  if ((s = gemm_common(precision, group_size, rank, M, N, K, act_codes, w_codes)) != SVDQ_OK) return s;
  if (M == 0) return ok();  // empty call: nothing to read or write
  if (!act_scales || !w_scales || !y) return fail(SVDQ_ERR_INVALID_ARG, "act_scales, w_scales and y are required");
  if ((rank > 0) != (xl1 != nullptr) || (rank > 0) != (l2t != nullptr))
    return fail(SVDQ_ERR_INVALID_ARG, "xl1 and l2t must be given iff rank > 0");
  if (precision == SVDQ_NVFP4 && !(act_global_scale > 0.0f && w_global_scale > 0.0f &&
                                   act_global_scale < 3.0e38f && w_global_scale < 3.0e38f))
    return fail(SVDQ_ERR_INVALID_ARG, "global scales must be finite and > 0 for nvfp4");
  // the epilogue applies the single factor fl32(alpha_a * alpha_w): it must be a
  // finite normal number, or y would come out inf, NaN or flushed
  if (precision == SVDQ_NVFP4) {
    const float prod = act_global_scale * w_global_scale;
    if (!(prod >= FLT_MIN && prod <= FLT_MAX))
      return fail(SVDQ_ERR_INVALID_ARG, "fl32(act_global_scale * w_global_scale) = %g is not a finite normal float",
                  (double)prod);
  }
  if (!aligned16(act_codes) || !aligned16(act_scales) || !aligned16(w_codes) || !aligned16(w_scales) ||
      !aligned16(xl1) || !aligned16(l2t) || !aligned16(bias) || !aligned16(y))
    return fail(SVDQ_ERR_ALIGNMENT, "all buffers must be 16-byte aligned");
  const size_t ny = (size_t)M * N * 2;
  const size_t ns_a = precision == SVDQ_INT4 ? (size_t)M * (K / 64) * 2 : (size_t)M * (K / 16);
  const size_t ns_w = precision == SVDQ_INT4 ? (size_t)N * (K / 64) * 2 : (size_t)N * (K / 16);
  if (overlaps(y, ny, act_codes, (size_t)M * K / 2) || overlaps(y, ny, w_codes, (size_t)N * K / 2) ||
      overlaps(y, ny, act_scales, ns_a) || overlaps(y, ny, w_scales, ns_w) ||
      overlaps(y, ny, xl1, (size_t)M * rank * 4) || overlaps(y, ny, l2t, (size_t)N * rank * 2) ||
      overlaps(y, ny, bias, (size_t)N * 2))
    return fail(SVDQ_ERR_INVALID_ARG, "y must not overlap an input");
  if (qkv) {
    const size_t nw = (size_t)qkv->head_dim * 2;
    if (!aligned16(qkv->norm_q) || !aligned16(qkv->norm_k) || !aligned16(qkv->rope))
      return fail(SVDQ_ERR_ALIGNMENT, "all buffers must be 16-byte aligned");
    if (overlaps(y, ny, qkv->norm_q, nw) || overlaps(y, ny, qkv->norm_k, nw) ||
        overlaps(y, ny, qkv->rope, rope_bytes))
      return fail(SVDQ_ERR_INVALID_ARG, "y must not overlap an input");
  }
  if ((s = check_arch()) != SVDQ_OK) return s;
  if (M == 0) return ok();
  if ((s = check_sticky()) != SVDQ_OK) return s;
  svdq::GemmArgs a{precision, rank, M, N, K, act_codes, act_scales, act_global_scale, w_codes,
                   w_scales, w_global_scale, xl1, l2t, bias, y, nullptr, qkv, nullptr, work};
  return launched(precision == SVDQ_INT4 ? svdq::launch_gemm_int4(a, (hipStream_t)stream)
                                         : svdq::launch_gemm_nvfp4(a, (hipStream_t)stream));
}

svdq_status svdq_w4a4_gemm(int precision, int group_size, int rank, int64_t M, int64_t N,
                           int64_t K, const void* act_codes, const void* act_scales,
                           float act_global_scale, const void* w_codes, const void* w_scales,
                           float w_global_scale, const float* xl1, const void* l2t,
                           const void* bias, void* y, void* stream) {
  return gemm_y(precision, group_size, rank, M, N, K, act_codes, act_scales, act_global_scale, w_codes,
                w_scales, w_global_scale, xl1, l2t, bias, y, stream, nullptr, 0);
}

static_assert(SVDQ_GEMM_WORK_BYTES == svdq::kGemmWorkBytes, "workspace size of the header and the kernels");

// The workspace of the split last round: NULL with work_bytes 0, or at least
// SVDQ_GEMM_WORK_BYTES, 16-byte aligned, overlapping no other buffer of the call.
static svdq_status check_work(void* work, int64_t work_bytes, int precision, int rank, int64_t M, int64_t N,
                              int64_t K, const void* act_codes, const void* act_scales, const void* w_codes,
                              const void* w_scales, const float* xl1, const void* l2t, const void* bias,
                              const void* y) {
  if (work) {
    if (work_bytes < (int64_t)SVDQ_GEMM_WORK_BYTES)
      return fail(SVDQ_ERR_INVALID_ARG, "work_bytes=%lld below SVDQ_GEMM_WORK_BYTES=%lld", (long long)work_bytes,
                  (long long)SVDQ_GEMM_WORK_BYTES);
    if (!aligned16(work)) return fail(SVDQ_ERR_ALIGNMENT, "all buffers must be 16-byte aligned");
    const size_t nw = SVDQ_GEMM_WORK_BYTES;
    const size_t ns_a = precision == SVDQ_INT4 ? (size_t)M * (K / 64) * 2 : (size_t)M * (K / 16);
    const size_t ns_w = precision == SVDQ_INT4 ? (size_t)N * (K / 64) * 2 : (size_t)N * (K / 16);
    if (M >= 0 && N > 0 && K > 0 && M <= kMaxDim && N <= kMaxDim && K <= kMaxDim && rank >= 0 && rank <= 128 &&
        (overlaps(work, nw, y, (size_t)M * N * 2) || overlaps(work, nw, act_codes, (size_t)M * K / 2) ||
         overlaps(work, nw, w_codes, (size_t)N * K / 2) || overlaps(work, nw, act_scales, ns_a) ||
         overlaps(work, nw, w_scales, ns_w) || overlaps(work, nw, xl1, (size_t)M * rank * 4) ||
         overlaps(work, nw, l2t, (size_t)N * rank * 2) || overlaps(work, nw, bias, (size_t)N * 2)))
      return fail(SVDQ_ERR_INVALID_ARG, "work must not overlap y or an input");
  } else if (work_bytes != 0) {
    return fail(SVDQ_ERR_INVALID_ARG, "work_bytes=%lld given without work", (long long)work_bytes);
  }
  return SVDQ_OK;
}

svdq_status svdq_w4a4_gemm_ws(int precision, int group_size, int rank, int64_t M, int64_t N,
                              int64_t K, const void* act_codes, const void* act_scales,
                              float act_global_scale, const void* w_codes, const void* w_scales,
                              float w_global_scale, const float* xl1, const void* l2t,
                              const void* bias, void* y, void* work, int64_t work_bytes, void* stream) {
  svdq_status s;
  if ((s = check_work(work, work_bytes, precision, rank, M, N, K, act_codes, act_scales, w_codes, w_scales, xl1,
                      l2t, bias, y)) != SVDQ_OK)
    return s;
  return gemm_y(precision, group_size, rank, M, N, K, act_codes, act_scales, act_global_scale, w_codes,
                w_scales, w_global_scale, xl1, l2t, bias, y, stream, nullptr, 0, work);
}

static svdq_status qkv_common(int precision, int group_size, int rank, int64_t M, int heads, int head_dim,
                              int64_t K, const void* act_codes, const void* act_scales, float act_global_scale,
                              const void* w_codes, const void* w_scales, float w_global_scale, const float* xl1,
                              const void* l2t, const void* bias, const void* norm_q, const void* norm_k, float eps,
                              const float* rope, int64_t rope_rows, void* y, void* work, int64_t work_bytes,
                              void* stream) {
  if (head_dim != 64 && head_dim != 128)
    return fail(SVDQ_ERR_UNSUPPORTED, "head_dim %d not in {64, 128}", head_dim);
  if (heads <= 0 || heads > (1 << 20)) return fail(SVDQ_ERR_INVALID_ARG, "bad head count %d", heads);
  const int64_t N = 3 * (int64_t)heads * head_dim;
  if (N % 128 != 0)
    return fail(SVDQ_ERR_UNSUPPORTED, "3 * heads * head_dim = %lld must be a multiple of 128", (long long)N);
  if (!(eps >= 0.0f && eps < 3.0e38f)) return fail(SVDQ_ERR_INVALID_ARG, "eps must be finite and >= 0");
  if (rope && (rope_rows <= 0 || rope_rows > kMaxDim))
    return fail(SVDQ_ERR_INVALID_ARG, "rope_rows must be >= 1 when rope is given");
  if (M > 0 && (!norm_q || !norm_k)) return fail(SVDQ_ERR_INVALID_ARG, "norm_q and norm_k are required");
  const svdq::QkvEpi q{(int)(heads * head_dim), head_dim, (const uint16_t*)norm_q, (const uint16_t*)norm_k,
                       eps, rope, rope ? (int)rope_rows : 1};
  const size_t rope_bytes = rope ? (size_t)rope_rows * head_dim * 4 : 0;
  svdq_status s;
  if ((s = check_work(work, work_bytes, precision, rank, M, N, K, act_codes, act_scales, w_codes, w_scales, xl1,
                      l2t, bias, y)) != SVDQ_OK)
    return s;
  if (work && (overlaps(work, SVDQ_GEMM_WORK_BYTES, norm_q, (size_t)head_dim * 2) ||
               overlaps(work, SVDQ_GEMM_WORK_BYTES, norm_k, (size_t)head_dim * 2) ||
               overlaps(work, SVDQ_GEMM_WORK_BYTES, rope, rope_bytes)))
    return fail(SVDQ_ERR_INVALID_ARG, "work must not overlap y or an input");
  return gemm_y(precision, group_size, rank, M, N, K, act_codes, act_scales, act_global_scale, w_codes,
                w_scales, w_global_scale, xl1, l2t, bias, y, stream, &q, rope_bytes, work);
}

svdq_status svdq_w4a4_gemm_qkv_norm_rope(int precision, int group_size, int rank, int64_t M,
                                         int heads, int head_dim, int64_t K, const void* act_codes,
                                         const void* act_scales, float act_global_scale,
                                         const void* w_codes, const void* w_scales,
                                         float w_global_scale, const float* xl1, const void* l2t,
                                         const void* bias, const void* norm_q, const void* norm_k,
                                         float eps, const float* rope, int64_t rope_rows, void* y,
                                         void* stream) {
  return qkv_common(precision, group_size, rank, M, heads, head_dim, K, act_codes, act_scales, act_global_scale,
                    w_codes, w_scales, w_global_scale, xl1, l2t, bias, norm_q, norm_k, eps, rope, rope_rows, y,
                    nullptr, 0, stream);
}

svdq_status svdq_w4a4_gemm_qkv_norm_rope_ws(int precision, int group_size, int rank, int64_t M,
                                            int heads, int head_dim, int64_t K, const void* act_codes,
                                            const void* act_scales, float act_global_scale,
                                            const void* w_codes, const void* w_scales,
                                            float w_global_scale, const float* xl1, const void* l2t,
                                            const void* bias, const void* norm_q, const void* norm_k,
                                            float eps, const float* rope, int64_t rope_rows, void* y,
                                            void* work, int64_t work_bytes, void* stream) {
  return qkv_common(precision, group_size, rank, M, heads, head_dim, K, act_codes, act_scales, act_global_scale,
                    w_codes, w_scales, w_global_scale, xl1, l2t, bias, norm_q, norm_k, eps, rope, rope_rows, y,
                    work, work_bytes, stream);
}

svdq_status svdq_w4a4_gemm_gelu_quant(int precision, int group_size, int rank, int64_t M, int64_t N,
                                     int64_t K, const void* act_codes, const void* act_scales,
                                     float act_global_scale, const void* w_codes, const void* w_scales,
                                     float w_global_scale, const float* xl1, const void* l2t,
                                     const void* bias, const void* smooth_out, const void* l1t_out,
                                     int rank_out, float out_global_scale, void* codes_out, void* scales_out,
                                     float* xl1_out, void* stream) {
  svdq_status s;
  if ((s = gemm_common(precision, group_size, rank, M, N, K, act_codes, w_codes)) != SVDQ_OK) return s;
  if (!valid_rank(rank_out)) return fail(SVDQ_ERR_UNSUPPORTED, "rank_out %d not in {0, 16, ..., 128}", rank_out);
  if (M * rank_out * 4 >= kMax32) return fail(SVDQ_ERR_UNSUPPORTED, "M*rank_out*4 must stay below 2^31 bytes");
  const bool fp4 = precision == SVDQ_NVFP4;
  if (fp4) {
    if (!(act_global_scale > 0.0f && w_global_scale > 0.0f && act_global_scale < 3.0e38f &&
          w_global_scale < 3.0e38f && out_global_scale > 0.0f && out_global_scale < 3.0e38f))
      return fail(SVDQ_ERR_INVALID_ARG, "global scales must be finite and > 0 for nvfp4");
    const float prod = act_global_scale * w_global_scale, d6 = 6.0f * out_global_scale;
    if (!(prod >= FLT_MIN && prod <= FLT_MAX))
      return fail(SVDQ_ERR_INVALID_ARG, "fl32(act_global_scale * w_global_scale) = %g is not a finite normal float",
                  (double)prod);
    if (!(d6 >= FLT_MIN && d6 <= FLT_MAX))
      return fail(SVDQ_ERR_INVALID_ARG, "fl32(6 * out_global_scale) = %g is not a finite normal float", (double)d6);
  }
  if (M == 0) return ok();
  if (!act_scales || !w_scales || !codes_out || !scales_out)
    return fail(SVDQ_ERR_INVALID_ARG, "act_scales, w_scales, codes_out and scales_out are required");
  if ((rank > 0) != (xl1 != nullptr) || (rank > 0) != (l2t != nullptr))
    return fail(SVDQ_ERR_INVALID_ARG, "xl1 and l2t must be given iff rank > 0");
  if ((rank_out > 0) != (l1t_out != nullptr) || (rank_out > 0) != (xl1_out != nullptr))
    return fail(SVDQ_ERR_INVALID_ARG, "l1t_out and xl1_out must be given iff rank_out > 0");
  if (!aligned16(act_codes) || !aligned16(act_scales) || !aligned16(w_codes) || !aligned16(w_scales) ||
      !aligned16(xl1) || !aligned16(l2t) || !aligned16(bias) || !aligned16(smooth_out) ||
      !aligned16(l1t_out) || !aligned16(codes_out) || !aligned16(scales_out) || !aligned16(xl1_out))
    return fail(SVDQ_ERR_ALIGNMENT, "all buffers must be 16-byte aligned");
  const size_t nc = (size_t)M * N / 2, nx = (size_t)M * rank_out * 4;
  const size_t ns = fp4 ? (size_t)M * (N / 16) : (size_t)M * (N / 64) * 2;
  const size_t ns_a = fp4 ? (size_t)M * (K / 16) : (size_t)M * (K / 64) * 2;
  const size_t ns_w = fp4 ? (size_t)N * (K / 16) : (size_t)N * (K / 64) * 2;
  const void* ins[] = {act_codes, act_scales, w_codes, w_scales, xl1, l2t, bias, smooth_out, l1t_out};
  const size_t nin[] = {(size_t)M * K / 2, ns_a, (size_t)N * K / 2, ns_w,
                        (size_t)M * rank * 4, (size_t)N * rank * 2, (size_t)N * 2, (size_t)N * 2,
                        (size_t)rank_out * N * 2};
  for (int i = 0; i < 9; ++i)
    if (overlaps(codes_out, nc, ins[i], nin[i]) || overlaps(scales_out, ns, ins[i], nin[i]) ||
        overlaps(xl1_out, nx, ins[i], nin[i]))
      return fail(SVDQ_ERR_INVALID_ARG, "outputs must not overlap an input");
  if (overlaps(codes_out, nc, scales_out, ns) || overlaps(codes_out, nc, xl1_out, nx) ||
      overlaps(scales_out, ns, xl1_out, nx))
    return fail(SVDQ_ERR_INVALID_ARG, "outputs must not overlap each other");
  if ((s = check_arch()) != SVDQ_OK) return s;
  if ((s = check_sticky()) != SVDQ_OK) return s;
  const svdq::MlpEpi me{(const uint16_t*)smooth_out, (const uint16_t*)l1t_out, rank_out, (uint8_t*)codes_out,
                        scales_out, xl1_out, fp4 ? out_global_scale : 1.0f};
  svdq::GemmArgs a{precision, rank, M, N, K, act_codes, act_scales, fp4 ? act_global_scale : 1.0f, w_codes,
                   w_scales, fp4 ? w_global_scale : 1.0f, xl1, l2t, bias, nullptr, nullptr, nullptr, &me};
  return launched(fp4 ? svdq::launch_gemm_nvfp4(a, (hipStream_t)stream) : svdq::launch_gemm_int4(a, (hipStream_t)stream));
}

svdq_status svdq_w4a4_group_psums(int precision, int group_size, int64_t M, int64_t N, int64_t K,
                                  const void* act_codes, const void* w_codes, void* psums,
                                  void* stream) {
  svdq_status s;
  if ((s = gemm_common(precision, group_size, 0, M, N, K, act_codes, w_codes)) != SVDQ_OK) return s;
  if (M == 0) return ok();  // empty call: nothing to read or write
  if (!psums) return fail(SVDQ_ERR_INVALID_ARG, "psums is required");
  if (!aligned16(act_codes) || !aligned16(w_codes) || !aligned16(psums))
    return fail(SVDQ_ERR_ALIGNMENT, "all buffers must be 16-byte aligned");
  const size_t np = (size_t)M * N * (K / group_size) * 4;
  if (overlaps(psums, np, act_codes, (size_t)M * K / 2) || overlaps(psums, np, w_codes, (size_t)N * K / 2))
    return fail(SVDQ_ERR_INVALID_ARG, "psums must not overlap an input");
  if ((s = check_arch()) != SVDQ_OK) return s;
  if (M == 0) return ok();
  if ((s = check_sticky()) != SVDQ_OK) return s;
  svdq::GemmArgs a{precision, 0, M, N, K, act_codes, nullptr, 1.0f, w_codes, nullptr, 1.0f,
                   nullptr, nullptr, nullptr, nullptr, psums, nullptr, nullptr};
  return launched(precision == SVDQ_INT4 ? svdq::launch_gemm_int4(a, (hipStream_t)stream)
                                         : svdq::launch_gemm_nvfp4(a, (hipStream_t)stream));
}

svdq_status svdq_calibrate_smooth(int64_t Mc, int64_t N, int64_t K, const void* x_cal, const void* w,
                                  void* smooth_out, void* stream) {
  if (Mc < 0 || N < 0 || K <= 0 || Mc > kMaxDim || N > kMaxDim || K > kMaxDim || K % 2 != 0)
    return fail(SVDQ_ERR_INVALID_ARG, "bad shape Mc=%lld N=%lld K=%lld", (long long)Mc, (long long)N, (long long)K);
  if (Mc * K > ((int64_t)1 << 31) || N * K > ((int64_t)1 << 31)) return fail(SVDQ_ERR_UNSUPPORTED, "operand above 2^31 elements");
  if (!smooth_out || (Mc > 0 && !x_cal) || (N > 0 && !w))
    return fail(SVDQ_ERR_INVALID_ARG, "x_cal, w and smooth_out are required");
  if (!aligned16(x_cal) || !aligned16(w) || !aligned16(smooth_out))
    return fail(SVDQ_ERR_ALIGNMENT, "all buffers must be 16-byte aligned");
  if (overlaps(smooth_out, (size_t)K * 2, x_cal, (size_t)Mc * K * 2) || overlaps(smooth_out, (size_t)K * 2, w, (size_t)N * K * 2))
    return fail(SVDQ_ERR_INVALID_ARG, "smooth_out must not overlap an input");
  svdq_status s;
  if ((s = check_arch()) != SVDQ_OK) return s;
  if ((s = check_sticky()) != SVDQ_OK) return s;
  return launched(svdq::launch_calibrate(Mc, N, K, x_cal, w, smooth_out, (hipStream_t)stream));
}

int64_t svdq_lowrank_workspace_bytes(int64_t N, int64_t K, int rank, int oversample) {
  if (N <= 0 || K <= 0 || rank <= 0 || oversample < 0 || rank + oversample > 64) return -1;
  return (int64_t)svdq::lowrank_workspace_bytes(N, K, rank + oversample);
}

static svdq_status lowrank_common(int64_t N, int64_t K, int rank, int oversample, int iters, const void* w,
                                  const void* smooth, const float* omega, void* l1t, void* l2t, float* residual,
                                  void* work, int64_t work_bytes, void* stream) {
  if (N <= 0 || K <= 0 || N > kMaxDim || K > kMaxDim || K % 64 != 0)
    return fail(SVDQ_ERR_INVALID_ARG, "bad shape N=%lld K=%lld (K %% 64 == 0)", (long long)N, (long long)K);
  if (N * K > ((int64_t)1 << 31)) return fail(SVDQ_ERR_UNSUPPORTED, "N*K above 2^31");
  if (rank <= 0 || rank % 16 != 0 || rank > 64 || oversample < 0 || rank + oversample > 64 ||
      rank + oversample > N || rank + oversample > K)
    return fail(SVDQ_ERR_UNSUPPORTED, "rank %d (multiple of 16) + oversample %d must be <= 64 and <= min(N, K)",
                rank, oversample);
  if (iters < 0 || iters > 64) return fail(SVDQ_ERR_INVALID_ARG, "iters %d not in [0, 64]", iters);
  if (!w || !omega || !l1t || !l2t || !residual)
    return fail(SVDQ_ERR_INVALID_ARG, "w, omega, l1t, l2t and residual are required");
  const bool noalloc = work == nullptr && work_bytes < 0;  // the allocation-free entry
  if (!work && !noalloc) return fail(SVDQ_ERR_INVALID_ARG, "work is required");
  const int p = rank + oversample;
  const int64_t need = (int64_t)svdq::lowrank_workspace_bytes(N, K, p);
  if (noalloc) {
    if (need > (int64_t)svdq::kNoAllocScratchBytes)
      return fail(SVDQ_ERR_UNSUPPORTED, "workspace of %lld bytes above the allocation-free limit of %lld bytes",
                  (long long)need, (long long)svdq::kNoAllocScratchBytes);
  } else if (work_bytes < need) {
    return fail(SVDQ_ERR_INVALID_ARG, "work_bytes %lld below svdq_lowrank_workspace_bytes()", (long long)work_bytes);
  }
  if (!aligned16(w) || !aligned16(smooth) || !aligned16(omega) || !aligned16(l1t) || !aligned16(l2t) ||
      !aligned16(residual) || !aligned16(work))
    return fail(SVDQ_ERR_ALIGNMENT, "all buffers must be 16-byte aligned");
  const size_t nr = (size_t)N * K * 4, nw = noalloc ? 0 : (size_t)work_bytes, n1 = (size_t)rank * K * 2, n2 = (size_t)N * rank * 2;
  const void* outs[] = {l1t, l2t, residual, work};
  const size_t nouts[] = {n1, n2, nr, nw};
  const void* ins[] = {w, smooth, omega};
  const size_t nins[] = {(size_t)N * K * 2, (size_t)K * 2, (size_t)K * p * 4};
  for (int i = 0; i < 4; ++i) {
    for (int j = 0; j < 3; ++j)
      if (overlaps(outs[i], nouts[i], ins[j], nins[j])) return fail(SVDQ_ERR_INVALID_ARG, "outputs must not overlap an input");
    for (int j = i + 1; j < 4; ++j)
      if (overlaps(outs[i], nouts[i], outs[j], nouts[j])) return fail(SVDQ_ERR_INVALID_ARG, "outputs must not overlap each other");
  }
  svdq_status s;
  if ((s = check_arch()) != SVDQ_OK) return s;
  if ((s = check_sticky()) != SVDQ_OK) return s;
  if (noalloc) {
    const hipError_t e = svdq::noalloc_scratch(&work);
    if (e != hipSuccess) return fail(SVDQ_ERR_DEVICE, "scratch address: %s", hipGetErrorString(e));
  }
  svdq::LowrankArgs a{N, K, rank, p, iters, w, smooth, omega, l1t, l2t, residual, work};
  return launched(svdq::launch_lowrank(a, (hipStream_t)stream));
}

svdq_status svdq_lowrank_decompose(int64_t N, int64_t K, int rank, int oversample, int iters, const void* w,
                                   const void* smooth, const float* omega, void* l1t, void* l2t, float* residual,
                                   void* work, int64_t work_bytes, void* stream) {
  if (!work) return fail(SVDQ_ERR_INVALID_ARG, "work is required");
  if (work_bytes < 0) return fail(SVDQ_ERR_INVALID_ARG, "work_bytes must be >= 0");
  return lowrank_common(N, K, rank, oversample, iters, w, smooth, omega, l1t, l2t, residual, work, work_bytes,
                        stream);
}

svdq_status svdq_lowrank_decompose_noalloc(int64_t N, int64_t K, int rank, int oversample, int iters,
                                           const void* w, const void* smooth, const float* omega, void* l1t,
                                           void* l2t, float* residual, void* stream) {
  return lowrank_common(N, K, rank, oversample, iters, w, smooth, omega, l1t, l2t, residual, nullptr, -1, stream);
}

svdq_status svdq_quantize_weight(int precision, int group_size, int64_t N, int64_t K, const float* residual,
                                 float w_global_scale, void* codes, void* scales, void* stream) {
  svdq_status s;
  if ((s = check_precision(precision, group_size)) != SVDQ_OK) return s;
  if (N < 0 || K <= 0 || N > kMaxDim || K > kMaxDim || K % 64 != 0)
    return fail(SVDQ_ERR_INVALID_ARG, "bad shape N=%lld K=%lld (K %% 64 == 0)", (long long)N, (long long)K);
  if (N * K > ((int64_t)1 << 31)) return fail(SVDQ_ERR_UNSUPPORTED, "N*K above 2^31");
  if (precision == SVDQ_NVFP4 && !(w_global_scale > 0.0f && w_global_scale < 3.0e38f))
    return fail(SVDQ_ERR_INVALID_ARG, "w_global_scale must be finite and > 0 for nvfp4");
  if (N == 0) return ok();
  if (!residual || !codes || !scales) return fail(SVDQ_ERR_INVALID_ARG, "residual, codes and scales are required");
  if (!aligned16(residual) || !aligned16(codes) || !aligned16(scales))
    return fail(SVDQ_ERR_ALIGNMENT, "all buffers must be 16-byte aligned");
  const size_t nr = (size_t)N * K * 4, nc = (size_t)N * K / 2;
  const size_t ns = precision == SVDQ_INT4 ? (size_t)N * (K / 64) * 2 : (size_t)N * (K / 16);
  if (overlaps(codes, nc, residual, nr) || overlaps(scales, ns, residual, nr) || overlaps(codes, nc, scales, ns))
    return fail(SVDQ_ERR_INVALID_ARG, "outputs must not overlap each other or the input");
  if ((s = check_arch()) != SVDQ_OK) return s;
  if ((s = check_sticky()) != SVDQ_OK) return s;
  return launched(svdq::launch_quantize_weight(precision, N, K, residual, w_global_scale, codes, scales,
                                               (hipStream_t)stream));
}

svdq_status awq_quantize_weight(int group_size, int64_t N, int64_t K, const void* w, void* codes, void* scales,
                                void* zeros, void* stream) {
  if (group_size != 64)
    return fail(SVDQ_ERR_UNSUPPORTED, "awq_w4a16 supports int4 with group 64; got group %d", group_size);
  if (N < 0 || K <= 0 || N > kMaxDim || K > kMaxDim || K % 64 != 0)
    return fail(SVDQ_ERR_INVALID_ARG, "bad shape N=%lld K=%lld (K %% 64 == 0)", (long long)N, (long long)K);
  if (N * K > ((int64_t)1 << 31)) return fail(SVDQ_ERR_UNSUPPORTED, "N*K above 2^31");
  if (N == 0) return ok();
  if (!w || !codes || !scales || !zeros) return fail(SVDQ_ERR_INVALID_ARG, "w, codes, scales and zeros are required");
  if (!aligned16(w) || !aligned16(codes) || !aligned16(scales) || !aligned16(zeros))
    return fail(SVDQ_ERR_ALIGNMENT, "all buffers must be 16-byte aligned");
  const size_t nw = (size_t)N * K * 2, nc = (size_t)N * K / 2, ng = (size_t)N * (K / 64) * 2;
  if (overlaps(codes, nc, w, nw) || overlaps(scales, ng, w, nw) || overlaps(zeros, ng, w, nw) ||
      overlaps(codes, nc, scales, ng) || overlaps(codes, nc, zeros, ng) || overlaps(scales, ng, zeros, ng))
    return fail(SVDQ_ERR_INVALID_ARG, "outputs must not overlap each other or the input");
  svdq_status s;
  if ((s = check_arch()) != SVDQ_OK) return s;
  if ((s = check_sticky()) != SVDQ_OK) return s;
  return launched(svdq::launch_awq_quantize(N, K, w, codes, scales, zeros, (hipStream_t)stream));
}

}  // extern "C"

// Validates an AWQ call; launches it, or with `prep` only fills *prep (left
// untouched for an empty call).
static svdq_status awq_gemv(int group_size, int64_t M, int64_t N, int64_t K, const void* x, const void* w_codes,
                            const void* w_scales, const void* w_zeros, const void* bias, void* y, void* stream,
                            svdq::AwqArgs* prep = nullptr) {
  if (group_size != 64)
    return fail(SVDQ_ERR_UNSUPPORTED, "awq_w4a16 supports int4 with group 64; got group %d", group_size);
  if (M < 0 || N <= 0 || K <= 0 || N > kMaxDim || K > kMaxDim)
    return fail(SVDQ_ERR_INVALID_ARG, "bad shape M=%lld N=%lld K=%lld", (long long)M, (long long)N, (long long)K);
  if (M > 64) return fail(SVDQ_ERR_UNSUPPORTED, "M=%lld above 64 (weight-only path is for small M)", (long long)M);
  if (K % 64 != 0) return fail(SVDQ_ERR_UNSUPPORTED, "K=%lld must be a multiple of 64", (long long)K);
  if (N % 64 != 0) return fail(SVDQ_ERR_UNSUPPORTED, "N=%lld must be a multiple of 64", (long long)N);
  if (N * K > ((int64_t)1 << 31)) return fail(SVDQ_ERR_UNSUPPORTED, "N*K above 2^31");
  if (M * K >= ((int64_t)1 << 30)) return fail(SVDQ_ERR_UNSUPPORTED, "M*K above 2^30 - 1 (x must stay below 2 GiB)");
  if (M == 0) return ok();  // empty call: nothing to read or write
  if (!x || !w_codes || !w_scales || !w_zeros || !y)
    return fail(SVDQ_ERR_INVALID_ARG, "x, w_codes, w_scales, w_zeros and y are required");
  if (!aligned16(x) || !aligned16(w_codes) || !aligned16(w_scales) || !aligned16(w_zeros) ||
      !aligned16(bias) || !aligned16(y))
    return fail(SVDQ_ERR_ALIGNMENT, "all buffers must be 16-byte aligned");
  const size_t ny = (size_t)M * N * 2, ng = (size_t)N * (K / 64) * 2;
  if (overlaps(y, ny, x, (size_t)M * K * 2) || overlaps(y, ny, w_codes, (size_t)N * K / 2) ||
      overlaps(y, ny, w_scales, ng) || overlaps(y, ny, w_zeros, ng) || overlaps(y, ny, bias, (size_t)N * 2))
    return fail(SVDQ_ERR_INVALID_ARG, "y must not overlap an input");
  svdq::AwqArgs a{M, N, K, x, w_codes, w_scales, w_zeros, bias, y};
  if (prep) {  // the caller checks the device once for both of its jobs
    *prep = a;
    return ok();
  }
  svdq_status s;
  if ((s = check_arch()) != SVDQ_OK) return s;
  if ((s = check_sticky()) != SVDQ_OK) return s;
  return launched(svdq::launch_awq(a, (hipStream_t)stream));
}

extern "C" {

svdq_status awq_w4a16_gemv(int group_size, int64_t M, int64_t N, int64_t K, const void* x,
                           const void* w_codes, const void* w_scales, const void* w_zeros,
                           const void* bias, void* y, void* stream) {
  return awq_gemv(group_size, M, N, K, x, w_codes, w_scales, w_zeros, bias, y, stream);
}

svdq_status svdq_quantize_act_awq_gemv(int precision, int group_size, int rank, int64_t M, int64_t K,
                                       const void* x, const void* smooth, const void* l1t,
                                       float act_global_scale, void* act_codes, void* act_scales, float* xl1,
                                       int awq_group_size, int64_t awq_M, int64_t awq_N, int64_t awq_K,
                                       const void* awq_x, const void* w_codes, const void* w_scales,
                                       const void* w_zeros, const void* bias, void* y, void* stream) {
  svdq::QuantArgs q{};
  svdq::AwqArgs w{};
  q.M = -1;
  w.M = -1;
  svdq_status s;
  if ((s = quantize_act(precision, group_size, rank, M, K, x, smooth, l1t, act_global_scale, act_codes, act_scales,
                        xl1, stream, nullptr, 0, &q)) != SVDQ_OK)
    return s;
  if ((s = awq_gemv(awq_group_size, awq_M, awq_N, awq_K, awq_x, w_codes, w_scales, w_zeros, bias, y, stream, &w)) !=
      SVDQ_OK)
    return s;
  const bool hq = q.M > 0, hw = w.M > 0;
  if (hq && hw) {  // the two jobs must not touch each other's outputs
    const size_t nc = (size_t)M * K / 2, nl = (size_t)M * rank * 4;
    const size_t ns = precision == SVDQ_INT4 ? (size_t)M * (K / 64) * 2 : (size_t)M * (K / 16);
    const size_t ny = (size_t)awq_M * awq_N * 2, ng = (size_t)awq_N * (awq_K / 64) * 2;
    const void* qin[3] = {x, smooth, l1t};
    const size_t qin_n[3] = {(size_t)M * K * 2, (size_t)K * 2, (size_t)rank * K * 2};
    const void* qout[3] = {act_codes, act_scales, xl1};
    const size_t qout_n[3] = {nc, ns, nl};
    const void* win[5] = {awq_x, w_codes, w_scales, w_zeros, bias};
    const size_t win_n[5] = {(size_t)awq_M * awq_K * 2, (size_t)awq_N * awq_K / 2, ng, ng, (size_t)awq_N * 2};
    for (int i = 0; i < 3; ++i)
      if (overlaps(y, ny, qin[i], qin_n[i]) || overlaps(y, ny, qout[i], qout_n[i]))
        return fail(SVDQ_ERR_INVALID_ARG, "the AWQ output must not overlap the quantizer's buffers");
    for (int i = 0; i < 3; ++i)
      for (int j = 0; j < 5; ++j)
        if (overlaps(qout[i], qout_n[i], win[j], win_n[j]))
          return fail(SVDQ_ERR_INVALID_ARG, "the quantizer's outputs must not overlap the AWQ inputs");
  }
  if (!hq && !hw) return ok();  // both empty: nothing to read or write (as for the two calls)
  if ((s = check_arch()) != SVDQ_OK) return s;
  if ((s = check_sticky()) != SVDQ_OK) return s;
  return launched(svdq::launch_quant_awq(hq ? &q : nullptr, hw ? &w : nullptr, (hipStream_t)stream));
}

}  // extern "C"
