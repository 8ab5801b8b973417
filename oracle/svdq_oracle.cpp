// Plain CPU oracle for the SVDQuant W4A4 linear layer and the AWQ W4A16
// weight-only linear.  TEST INFRASTRUCTURE ONLY: nothing on the product path
// may link, load or call this file.  It shares no code, header, table or
// constant with the HIP library; the two meet only at the byte layouts of the
// buffers they read and write.
//
// Sources (page titles and sections):
//  * "Nunchaku Lite" (Diffusers quantization docs), table in "Supported
//    quantization types": svdq_w4a4 comes as int4 with group 64 and as nvfp4
//    with group 16, both with a low-rank correction; awq_w4a16 is int4
//    weight-only with group 64.
//  * "Nunchaku Lite", "NunchakuLiteQuantizationConfig": the float buffers of a
//    quantized module run in compute_dtype (bfloat16).
//  * "Nunchaku 4-bit inference in Diffusers" (blog), "Background: SVDQuant and
//    Nunchaku": activation outliers are moved into the weights (smoothing),
//    a 16-bit low-rank branch carries the hardest part of each weight and the
//    residual runs as 4-bit weights x 4-bit activations; the low-rank
//    down-projection belongs with the activation quantizer and the up-
//    projection with the 4-bit GEMM.
//  * same blog, "Introducing Nunchaku Lite": awq_w4a16 serves memory-bound,
//    precision-sensitive modulation projections.
//
// The pages give no formulas.  Every numeric choice below is a reading,
// stated where it is made; each is a plain definition written out step by
// step.  All accumulation is in double; every value that the method stores
// in a narrow format is rounded with the generic round-to-nearest-even
// routine `round_to_format`.
//
// Build: g++ -O2 -ffp-contract=off -fno-fast-math -shared -fPIC -pthread
// (no FMA contraction, no reassociation: float ops round exactly as written).

#include <cmath>
#include <cstdint>
#include <cstring>
#include <thread>
#include <vector>
#include <algorithm>

namespace {

// ---------------------------------------------------------------------------
// Number formats.  A binary floating-point format is described by its number
// of explicit mantissa bits, its minimum normal exponent, and the largest
// finite magnitude.  round_to_format returns the nearest representable value
// of x (ties to even mantissa), with subnormals below the minimum normal
// exponent.  Magnitudes that round above the largest finite value either
// saturate to it or become infinity, as asked.
// ---------------------------------------------------------------------------
enum Special { kIeee, kFnNan, kNone };  // all-ones exponent: inf/NaN, NaN only at mantissa all-ones, or nothing

struct Fmt {
  int mant_bits;   // explicit mantissa bits
  int emin;        // exponent of the smallest normal number
  double maxv;     // largest finite magnitude
  Special special; // meaning of the top encodings
};

const Fmt kF16  = {10, -14, 65504.0, kIeee};
const Fmt kBF16 = {7, -126, 3.3895313892515355e38, kIeee};
const Fmt kE4M3 = {3, -6, 448.0, kFnNan};  // OCP E4M3 "FN": no infinities, max 448
const Fmt kE2M1 = {1, 0, 6.0, kNone};      // OCP E2M1: {0, .5, 1, 1.5, 2, 3, 4, 6}

double round_to_format(double x, const Fmt& f, bool saturate) {
  if (x == 0.0 || std::isnan(x)) return x;
  if (std::isinf(x)) return saturate ? std::copysign(f.maxv, x) : x;
  double a = std::fabs(x);
  int e;
  std::frexp(a, &e);          // a = m * 2^e, m in [0.5, 1)
  e -= 1;                     // a = m' * 2^e, m' in [1, 2)
  if (e < f.emin) e = f.emin; // subnormal range: fixed quantum
  double quantum = std::ldexp(1.0, e - f.mant_bits);
  double r = std::nearbyint(a / quantum) * quantum;  // RNE (default mode)
  if (r > f.maxv) r = saturate ? f.maxv : INFINITY;
  return std::copysign(r, x);
}

// Encode a value already representable in format f into its bit pattern
// (sign at bit 1 + exp_bits + mant_bits, exponent bias from emin).
uint32_t encode(double v, const Fmt& f, int exp_bits) {
  uint32_t sign = std::signbit(v) ? 1u : 0u;
  double a = std::fabs(v);
  uint32_t bits;
  int bias = 1 - f.emin;
  if (std::isnan(a)) {  // canonical NaN: all-ones exponent and mantissa
    return (sign << (exp_bits + f.mant_bits)) | ((1u << (exp_bits + f.mant_bits)) - 1u);
  } else if (std::isinf(a)) {
    bits = ((1u << exp_bits) - 1u) << f.mant_bits;
  } else if (a == 0.0) {
    bits = 0;
  } else {
    int e;
    std::frexp(a, &e);
    e -= 1;
    if (e < f.emin) {  // subnormal: mantissa counts quanta of 2^(emin-mant)
      bits = (uint32_t)std::ldexp(a, f.mant_bits - f.emin);
    } else {
      uint32_t m = (uint32_t)((std::ldexp(a, -e) - 1.0) * (double)(1u << f.mant_bits));
      bits = ((uint32_t)(e + bias) << f.mant_bits) | m;
    }
  }
  return (sign << (exp_bits + f.mant_bits)) | bits;
}

double decode(uint32_t bits, const Fmt& f, int exp_bits) {
  uint32_t mmask = (1u << f.mant_bits) - 1u;
  uint32_t m = bits & mmask;
  uint32_t ef = (bits >> f.mant_bits) & ((1u << exp_bits) - 1u);
  bool neg = (bits >> (exp_bits + f.mant_bits)) & 1u;
  int bias = 1 - f.emin;
  double v;
  uint32_t emax_field = (1u << exp_bits) - 1u;
  if (f.special == kIeee && ef == emax_field) v = m ? NAN : INFINITY;
  else if (f.special == kFnNan && ef == emax_field && m == mmask) v = NAN;
  else if (ef == 0) v = std::ldexp((double)m, f.emin - f.mant_bits);
  else v = std::ldexp(1.0 + (double)m / (double)(1u << f.mant_bits), (int)ef - bias);
  return neg ? -v : v;
}

inline float bf16_to_f32(uint16_t h) { return (float)decode(h, kBF16, 8); }
inline float f16_to_f32(uint16_t h) { return (float)decode(h, kF16, 5); }
inline float e4m3_to_f32(uint8_t b) { return (float)decode(b, kE4M3, 4); }
inline float e2m1_to_f32(uint8_t c) { return (float)decode(c & 0xF, kE2M1, 2); }

// fp16 with saturation at 65504 (scales never become infinite).
inline uint16_t f32_to_f16_sat(float x) {
  return (uint16_t)encode(round_to_format(x, kF16, true), kF16, 5);
}
inline uint16_t f32_to_bf16(float x) {
  return (uint16_t)encode(round_to_format(x, kBF16, false), kBF16, 8);
}
inline uint16_t f64_to_bf16(double x) {
  return (uint16_t)encode(round_to_format(x, kBF16, false), kBF16, 8);
}
inline uint8_t f32_to_e4m3_sat(float x) {
  return (uint8_t)encode(round_to_format(x, kE4M3, true), kE4M3, 4);
}
// E2M1 keeps the sign of its input, also when the magnitude rounds to zero.
inline uint8_t f32_to_e2m1_sat(float x) {
  return (uint8_t)encode(round_to_format(x, kE2M1, true), kE2M1, 2);
}

// Two's-complement nibble of a code in [-8, 7].
inline int nibble_to_int(uint8_t n) { return (n & 8) ? (int)(n & 0xF) - 16 : (int)(n & 0xF); }
inline uint8_t get_nibble(const uint8_t* row, int64_t k) {
  uint8_t b = row[k >> 1];
  return (k & 1) ? (uint8_t)(b >> 4) : (uint8_t)(b & 0xF);
}
inline void put_nibble(uint8_t* row, int64_t k, uint8_t n) {
  uint8_t& b = row[k >> 1];
  if (k & 1) b = (uint8_t)((b & 0x0F) | ((n & 0xF) << 4));
  else b = (uint8_t)((b & 0xF0) | (n & 0xF));
}

template <class F>
void parallel_rows(int64_t rows, int nthreads, F fn) {
  if (nthreads <= 0) nthreads = (int)std::max(1u, std::thread::hardware_concurrency());
  if (rows < 2 || nthreads == 1) { for (int64_t r = 0; r < rows; ++r) fn(r); return; }
  int64_t nt = std::min<int64_t>(nthreads, rows);
  std::vector<std::thread> pool;
  for (int64_t t = 0; t < nt; ++t) {
    pool.emplace_back([&, t]() { for (int64_t r = t; r < rows; r += nt) fn(r); });
  }
  for (auto& th : pool) th.join();
}

// Per-channel reciprocal of the smoothing factor lambda (bf16 [K]); NULL
// means lambda = 1.  Reading: the smoothed activation is formed as
// x * fl32(1/lambda_k), one IEEE division per channel.
std::vector<float> smoothing_reciprocals(int64_t K, const uint16_t* lam) {
  std::vector<float> r((size_t)K, 1.0f);
  if (lam) for (int64_t k = 0; k < K; ++k) r[k] = 1.0f / bf16_to_f32(lam[k]);
  return r;
}

}  // namespace

extern "C" {

// ---------------------------------------------------------------------------
// Converters, exported for the pin tests (each compared against a library
// routine over every 32-bit input).
// ---------------------------------------------------------------------------
void orc_vec_f32_to_f16_sat(const float* in, uint16_t* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = f32_to_f16_sat(in[i]);
}
void orc_vec_f32_to_bf16(const float* in, uint16_t* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = f32_to_bf16(in[i]);
}
void orc_vec_f32_to_e4m3_sat(const float* in, uint8_t* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = f32_to_e4m3_sat(in[i]);
}
void orc_vec_f32_to_e2m1_sat(const float* in, uint8_t* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = f32_to_e2m1_sat(in[i]);
}
void orc_vec_f16_to_f32(const uint16_t* in, float* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = f16_to_f32(in[i]);
}
void orc_vec_bf16_to_f32(const uint16_t* in, float* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = bf16_to_f32(in[i]);
}
void orc_vec_e4m3_to_f32(const uint8_t* in, float* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = e4m3_to_f32(in[i]);
}
void orc_vec_e2m1_to_f32(const uint8_t* in, float* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = e2m1_to_f32(in[i]);
}

// ---------------------------------------------------------------------------
// Activation quantization, int4 group 64 ("Supported quantization types"),
// applied to the smoothed activation X/lambda ("Background: SVDQuant and
// Nunchaku").  Per row m and group g of 64 channels:
//   xh_k  = fl32(x_k * fl32(1/lambda_k))
//   a     = max |xh_k|                       (exact)
//   s     = fp16_sat(fl32(a / 7))            qmax = 7 for signed int4
//   q_k   = 0 if s == 0, else clamp(rne(fl32(xh_k * fl32(1/s))), -8, 7)
// Codes are packed two per byte, even channel in the low nibble, two's
// complement; scales are fp16 bits [M, K/64].
// ---------------------------------------------------------------------------
void orc_quantize_act_int4(int64_t M, int64_t K, const uint16_t* x, const uint16_t* lam,
                           uint8_t* codes, uint16_t* scales, int nthreads) {
  const int64_t G = 64, ng = K / G;
  std::vector<float> rl = smoothing_reciprocals(K, lam);
  parallel_rows(M, nthreads, [&](int64_t m) {
    const uint16_t* xr = x + m * K;
    uint8_t* cr = codes + m * (K / 2);
    std::vector<float> xh((size_t)G);
    for (int64_t g = 0; g < ng; ++g) {
      float a = 0.0f;
      for (int64_t j = 0; j < G; ++j) {
        int64_t k = g * G + j;
        xh[j] = bf16_to_f32(xr[k]) * rl[k];
        a = std::max(a, std::fabs(xh[j]));
      }
      uint16_t sbits = f32_to_f16_sat(a / 7.0f);
      scales[m * ng + g] = sbits;
      float s = f16_to_f32(sbits);
      float t = (s == 0.0f) ? 0.0f : 1.0f / s;
      for (int64_t j = 0; j < G; ++j) {
        int q = 0;
        if (s != 0.0f) {
          float v = xh[j] * t;
          float r = std::nearbyint(v);
          r = std::min(7.0f, std::max(-8.0f, r));
          q = (int)r;
        }
        put_nibble(cr, g * G + j, (uint8_t)(q & 0xF));
      }
    }
  });
}

// ---------------------------------------------------------------------------
// Activation quantization, NVFP4 group 16 ("Supported quantization types").
// NVFP4 = E2M1 values, one E4M3 scale per 16 channels, one fp32 per-tensor
// scale alpha (static, calibrated, passed in).  Per row m and group g:
//   xh_k = fl32(x_k * fl32(1/lambda_k)),  a = max |xh_k|
//   s    = e4m3_sat(fl32(a / fl32(6 * alpha)))     6 = largest E2M1 value
//   c_k  = 0x0 if s == 0, else e2m1_sat(fl32(xh_k * fl32(1 / fl32(s*alpha))))
// Codes: E2M1 nibbles, sign in bit 3, even channel low; scales: E4M3 bytes.
// ---------------------------------------------------------------------------
void orc_quantize_act_nvfp4(int64_t M, int64_t K, const uint16_t* x, const uint16_t* lam,
                            float alpha, uint8_t* codes, uint8_t* scales, int nthreads) {
  const int64_t G = 16, ng = K / G;
  std::vector<float> rl = smoothing_reciprocals(K, lam);
  const float d = 6.0f * alpha;
  parallel_rows(M, nthreads, [&](int64_t m) {
    const uint16_t* xr = x + m * K;
    uint8_t* cr = codes + m * (K / 2);
    float xh[16];
    for (int64_t g = 0; g < ng; ++g) {
      float a = 0.0f;
      for (int64_t j = 0; j < G; ++j) {
        int64_t k = g * G + j;
        xh[j] = bf16_to_f32(xr[k]) * rl[k];
        a = std::max(a, std::fabs(xh[j]));
      }
      uint8_t sbits = f32_to_e4m3_sat(a / d);
      scales[m * ng + g] = sbits;
      float s = e4m3_to_f32(sbits);
      float t = 0.0f;
      if (s != 0.0f) { float sa = s * alpha; t = 1.0f / sa; }
      for (int64_t j = 0; j < G; ++j) {
        uint8_t c = (s == 0.0f) ? (uint8_t)0 : f32_to_e2m1_sat(xh[j] * t);
        put_nibble(cr, g * G + j, c);
      }
    }
  });
}

// ---------------------------------------------------------------------------
// Low-rank down-projection XL1 = X . L1 on the raw bf16 X (the low-rank branch
// is stored in the form that consumes X, so X is read once by the quantizer),
// "Background: SVDQuant and Nunchaku" (down-projection fused with the
// quantizer).  L1 is given transposed, l1t = L1^T bf16 [r, K].  Double sums,
// stored as fp32 [M, r].
// ---------------------------------------------------------------------------
void orc_lowrank_down(int64_t M, int64_t K, int r, const uint16_t* x, const uint16_t* l1t,
                      float* xl1, int nthreads) {
  std::vector<double> l1d((size_t)(r * K));
  for (int64_t i = 0; i < (int64_t)r * K; ++i) l1d[i] = bf16_to_f32(l1t[i]);
  parallel_rows(M, nthreads, [&](int64_t m) {
    std::vector<double> xd((size_t)K);
    for (int64_t k = 0; k < K; ++k) xd[k] = bf16_to_f32(x[m * K + k]);
    for (int j = 0; j < r; ++j) {
      double acc = 0.0;
      const double* lr = &l1d[(size_t)j * K];
      for (int64_t k = 0; k < K; ++k) acc += xd[k] * lr[k];
      xl1[m * r + j] = (float)acc;
    }
  });
}

// ---------------------------------------------------------------------------
// Per-group partial sums of the 4-bit product, P[m, n, g] = sum over the
// group's channels of a_code * w_code.  int4: exact int32.  nvfp4: the sum of
// E2M1 products (multiples of 1/4, |P| <= 576), exact in fp32.  Output layout
// [M, N, K/G], g fastest.
// ---------------------------------------------------------------------------
void orc_group_psums(int prec, int64_t M, int64_t N, int64_t K, const uint8_t* a,
                     const uint8_t* w, void* psums, int nthreads) {
  const int64_t G = prec == 0 ? 64 : 16, ng = K / G;
  parallel_rows(M, nthreads, [&](int64_t m) {
    const uint8_t* ar = a + m * (K / 2);
    for (int64_t n = 0; n < N; ++n) {
      const uint8_t* wr = w + n * (K / 2);
      for (int64_t g = 0; g < ng; ++g) {
        if (prec == 0) {
          int64_t acc = 0;
          for (int64_t j = 0; j < G; ++j) {
            int64_t k = g * G + j;
            acc += (int64_t)nibble_to_int(get_nibble(ar, k)) * nibble_to_int(get_nibble(wr, k));
          }
          ((int32_t*)psums)[(m * N + n) * ng + g] = (int32_t)acc;
        } else {
          double acc = 0.0;
          for (int64_t j = 0; j < G; ++j) {
            int64_t k = g * G + j;
            acc += (double)e2m1_to_f32(get_nibble(ar, k)) * (double)e2m1_to_f32(get_nibble(wr, k));
          }
          ((float*)psums)[(m * N + n) * ng + g] = (float)acc;
        }
      }
    }
  });
}

// ---------------------------------------------------------------------------
// The quantized linear, one output at a time:
//   y[m,n] = sum_g sa[m,g] * sw[n,g] * P[m,n,g]            (int4)
//   y[m,n] = alpha_a * alpha_w * sum_g sa * sw * P          (nvfp4)
//          + sum_j XL1[m,j] * L2[j,n] + bias[n]
// all in double; L2 is given transposed, l2t = L2^T bf16 [N, r]; bias may be
// NULL; r may be 0.  Evaluated at the (rows[i], cols[i]) pairs when count >= 0,
// else over the full [M, N] grid (count = -1).  y_out gets the double result
// and y_bf16 (may be NULL) its bf16 rounding.
// ---------------------------------------------------------------------------
void orc_w4a4_linear(int prec, int r, int64_t M, int64_t N, int64_t K,
                     const uint8_t* a_codes, const void* a_scales, float alpha_a,
                     const uint8_t* w_codes, const void* w_scales, float alpha_w,
                     const float* xl1, const uint16_t* l2t, const uint16_t* bias,
                     int64_t count, const int64_t* rows, const int64_t* cols,
                     double* y_out, uint16_t* y_bf16, int nthreads) {
  const int64_t G = prec == 0 ? 64 : 16, ng = K / G;
  auto one = [&](int64_t m, int64_t n) -> double {
    const uint8_t* ar = a_codes + m * (K / 2);
    const uint8_t* wr = w_codes + n * (K / 2);
    double main = 0.0;
    for (int64_t g = 0; g < ng; ++g) {
      double P = 0.0, sa, sw;
      for (int64_t j = 0; j < G; ++j) {
        int64_t k = g * G + j;
        if (prec == 0)
          P += (double)nibble_to_int(get_nibble(ar, k)) * (double)nibble_to_int(get_nibble(wr, k));
        else
          P += (double)e2m1_to_f32(get_nibble(ar, k)) * (double)e2m1_to_f32(get_nibble(wr, k));
      }
      if (prec == 0) {
        sa = f16_to_f32(((const uint16_t*)a_scales)[m * ng + g]);
        sw = f16_to_f32(((const uint16_t*)w_scales)[n * ng + g]);
      } else {
        sa = e4m3_to_f32(((const uint8_t*)a_scales)[m * ng + g]);
        sw = e4m3_to_f32(((const uint8_t*)w_scales)[n * ng + g]);
      }
      main += sa * sw * P;
    }
    if (prec != 0) main *= (double)alpha_a * (double)alpha_w;
    double lr = 0.0;
    for (int j = 0; j < r; ++j) lr += (double)xl1[m * r + j] * (double)bf16_to_f32(l2t[n * r + j]);
    double b = bias ? (double)bf16_to_f32(bias[n]) : 0.0;
    return main + lr + b;
  };
  if (count < 0) {
    parallel_rows(M, nthreads, [&](int64_t m) {
      for (int64_t n = 0; n < N; ++n) {
        double v = one(m, n);
        y_out[m * N + n] = v;
        if (y_bf16) y_bf16[m * N + n] = f64_to_bf16(v);
      }
    });
  } else {
    parallel_rows(count, nthreads, [&](int64_t i) {
      double v = one(rows[i], cols[i]);
      y_out[i] = v;
      if (y_bf16) y_bf16[i] = f64_to_bf16(v);
    });
  }
}

// ---------------------------------------------------------------------------
// AWQ W4A16 ("Supported quantization types": int4 weight-only, group 64;
// "Introducing Nunchaku Lite": modulation projections).  Reading: unsigned
// codes q in 0..15 (even channel low nibble), fp16 scale s and fp16 zero-point
// z per (row n, group g), dequantized weight (q - z) * s:
//   y[m,n] = sum_g sum_{k in g} x[m,k] * (q[n,k] - z[n,g]) * s[n,g] + bias[n]
// in double; same sampled/full convention as orc_w4a4_linear.
// ---------------------------------------------------------------------------
void orc_awq_linear(int64_t M, int64_t N, int64_t K, const uint16_t* x, const uint8_t* w_codes,
                    const uint16_t* w_scales, const uint16_t* w_zeros, const uint16_t* bias,
                    int64_t count, const int64_t* rows, const int64_t* cols,
                    double* y_out, uint16_t* y_bf16, int nthreads) {
  const int64_t G = 64, ng = K / G;
  auto one = [&](int64_t m, int64_t n) -> double {
    const uint8_t* wr = w_codes + n * (K / 2);
    double acc = 0.0;
    for (int64_t g = 0; g < ng; ++g) {
      double s = f16_to_f32(w_scales[n * ng + g]);
      double z = f16_to_f32(w_zeros[n * ng + g]);
      for (int64_t j = 0; j < G; ++j) {
        int64_t k = g * G + j;
        double q = (double)get_nibble(wr, k);
        acc += (double)bf16_to_f32(x[m * K + k]) * (q - z) * s;
      }
    }
    if (bias) acc += (double)bf16_to_f32(bias[n]);
    return acc;
  };
  if (count < 0) {
    parallel_rows(M * N, nthreads, [&](int64_t i) {
      double v = one(i / N, i % N);
      y_out[i] = v;
      if (y_bf16) y_bf16[i] = f64_to_bf16(v);
    });
  } else {
    parallel_rows(count, nthreads, [&](int64_t i) {
      double v = one(rows[i], cols[i]);
      y_out[i] = v;
      if (y_bf16) y_bf16[i] = f64_to_bf16(v);
    });
  }
}

// ---------------------------------------------------------------------------
// Q/K/V epilogue of the fused attention projection (blog "Nunchaku 4-bit
// inference in Diffusers", "Quantizing models with structural rewrites": the
// Q, K and V projections are one linear whose output concatenates Q, K and V
// in that order, and one operator applies the projection, the Q and K
// normalizations and the rotary embedding; "Nunchaku Lite", "Fused kernels":
// the QKV + RMSNorm + RoPE fusion of the original engine).  The pages give
// the order of the steps (norm of Q and K, then the rotary embedding) but no
// formulas; readings, all in double:
//   * columns: [Q | K | V], each heads*D wide; head h of Q is columns
//     h*D .. h*D+D-1, of K the same plus heads*D; V is left as it is;
//   * RMSNorm of one head of one token: y_d * w_d / sqrt(mean_d(y_d^2) + eps),
//     w = norm_q (bf16 [D]) for Q heads, norm_k for K heads;
//   * rotary embedding, applied after the norm: channel pairs (2p, 2p+1) of
//     the head are rotated by the angle of table entry (s, p):
//     (a, b) -> (a*cos - b*sin, a*sin + b*cos), with (cos, sin) given as fp32
//     pairs in rope [S, D/2, 2]; token row m uses table row m mod S (rows are
//     batch-major [batch, S]).  rope == NULL: no rotation.
// y_in [rows, 3*heads*D] holds the projection (bias included) of the tokens
// row_ids[i]; y_out gets the result in double and y_bf16 (may be NULL) its
// bf16 rounding.
// ---------------------------------------------------------------------------
void orc_qkv_norm_rope(int64_t rows, int heads, int D, const double* y_in, const int64_t* row_ids,
                       const uint16_t* norm_q, const uint16_t* norm_k, double eps,
                       const float* rope, int64_t rope_rows, double* y_out, uint16_t* y_bf16) {
  const int64_t HD = (int64_t)heads * D, N = 3 * HD;
  std::vector<double> head(D);
  for (int64_t i = 0; i < rows; ++i) {
    const double* yi = y_in + i * N;
    double* yo = y_out + i * N;
    for (int64_t n = 0; n < N; ++n) yo[n] = yi[n];
    for (int part = 0; part < 2; ++part) {  // 0: Q, 1: K
      const uint16_t* w = part == 0 ? norm_q : norm_k;
      for (int h = 0; h < heads; ++h) {
        const int64_t c0 = part * HD + (int64_t)h * D;
        double ss = 0.0;
        for (int d = 0; d < D; ++d) ss += yi[c0 + d] * yi[c0 + d];
        const double inv = 1.0 / std::sqrt(ss / D + eps);
        for (int d = 0; d < D; ++d) head[d] = yi[c0 + d] * inv * (double)bf16_to_f32(w[d]);
        if (rope) {
          const int64_t s = row_ids[i] % rope_rows;
          for (int p = 0; p < D / 2; ++p) {
            const double c = rope[(s * (D / 2) + p) * 2], sn = rope[(s * (D / 2) + p) * 2 + 1];
            const double a = head[2 * p], b = head[2 * p + 1];
            head[2 * p] = a * c - b * sn;
            head[2 * p + 1] = a * sn + b * c;
          }
        }
        for (int d = 0; d < D; ++d) yo[c0 + d] = head[d];
      }
    }
    if (y_bf16)
      for (int64_t n = 0; n < N; ++n) y_bf16[i * N + n] = f64_to_bf16(yo[n]);
  }
}

// ---------------------------------------------------------------------------
// GELU of the diffusion-transformer MLP ("Nunchaku Lite", "Fused kernels":
// the original engine fuses the GELU MLP).  The pages name GELU without a
// formula; read as the exact form y * Phi(y) with Phi the standard normal
// CDF, written 0.5 * y * erfc(-y / sqrt(2)) (the same function as
// 0.5 * y * (1 + erf(y / sqrt(2))), without the cancellation for negative y),
// in double, then rounded once to bf16 (the compute dtype of the layer, the
// input format of the next quantizer).  h_bf16 may be NULL.
// ---------------------------------------------------------------------------
void orc_gelu(int64_t n, const double* y, double* h, uint16_t* h_bf16) {
  for (int64_t i = 0; i < n; ++i) {
    const double v = 0.5 * y[i] * std::erfc(-y[i] / std::sqrt(2.0));
    h[i] = v;
    if (h_bf16) h_bf16[i] = f64_to_bf16(v);
  }
}

// The smoothed activation the quantizer rounds, xh = fl32(x * fl32(1/lambda_k))
// (same arithmetic as the first step of orc_quantize_act_*), exported so that
// a check can see how far a value lies from a rounding boundary.
void orc_smooth(int64_t M, int64_t K, const uint16_t* x, const uint16_t* lam, float* xh) {
  std::vector<float> rl = smoothing_reciprocals(K, lam);
  for (int64_t m = 0; m < M; ++m)
    for (int64_t k = 0; k < K; ++k) xh[m * K + k] = bf16_to_f32(x[m * K + k]) * rl[k];
}

// ---------------------------------------------------------------------------
// Offline weight side of SVDQuant (blog "Nunchaku 4-bit inference in
// Diffusers", "Background: SVDQuant and Nunchaku": activation outliers are
// moved into the weights, the hardest part of each weight becomes a 16-bit
// low-rank branch, the residual is quantized to 4 bits; "Nunchaku Lite",
// quantization walkthrough: the checkpoint is produced offline from the dense
// weights).  The pages give no formulas; readings:
//   * smoothing factor per input channel k (SmoothQuant-style migration with
//     strength 1/2): lambda_k = bf16(sqrt(fl32(a_k / b_k))), a_k = max_m |X_mk|
//     over the calibration batch, b_k = max_n |W_nk|; 1 when a_k or b_k is 0;
//   * (the rank-r decomposition of the smoothed weight is computed in
//     oracle/__init__.py with numpy's SVD in double);
//   * residual quantization per (row n, group of G channels), int4 G = 64:
//       s = fp16_sat(fl32(amax / 7)), q = clamp(rne(fl32(r * fl32(1/s))), -8, 7)
//     nvfp4 G = 16 with the per-tensor scale alpha_w:
//       s = e4m3_sat(fl32(amax / fl32(6 alpha))), c = e2m1_sat(fl32(r * fl32(1/fl32(s alpha))))
//     i.e. the activation quantizer's steps on an fp32 input without smoothing;
//   * AWQ weights (int4 weight-only, group 64, unsigned codes with a zero-point):
//     min-max asymmetric quantization per (row, group) over a range that
//     contains 0 (so 0 is exact): lo = min(0, min w), hi = max(0, max w),
//     s = fp16(fl32((hi - lo) / 15)), z = clamp(rne(fl32(-lo * fl32(1/s))), 0, 15)
//     stored as fp16, q = clamp(rne(fl32(w * fl32(1/s))) + z, 0, 15); an
//     all-zero group has s = 0, z = 0, codes 0.
// ---------------------------------------------------------------------------
void orc_calibrate_smooth(int64_t Mc, int64_t N, int64_t K, const uint16_t* x, const uint16_t* w,
                          uint16_t* lam) {
  for (int64_t k = 0; k < K; ++k) {
    float a = 0.0f, b = 0.0f;
    for (int64_t m = 0; m < Mc; ++m) a = std::max(a, std::fabs(bf16_to_f32(x[m * K + k])));
    for (int64_t n = 0; n < N; ++n) b = std::max(b, std::fabs(bf16_to_f32(w[n * K + k])));
    float l = 1.0f;
    if (a > 0.0f && b > 0.0f) l = std::sqrt(a / b);
    lam[k] = f32_to_bf16(l);
  }
}

void orc_quantize_weight(int prec, int64_t N, int64_t K, const float* r, float alpha, uint8_t* codes,
                         void* scales) {
  const int64_t G = prec == 0 ? 64 : 16, ng = K / G;
  for (int64_t n = 0; n < N; ++n) {
    const float* rr = r + n * K;
    uint8_t* cr = codes + n * (K / 2);
    for (int64_t g = 0; g < ng; ++g) {
      float a = 0.0f;
      for (int64_t j = 0; j < G; ++j) a = std::max(a, std::fabs(rr[g * G + j]));
      if (prec == 0) {
        const uint16_t sbits = f32_to_f16_sat(a / 7.0f);
        ((uint16_t*)scales)[n * ng + g] = sbits;
        const float s = f16_to_f32(sbits);
        const float t = s == 0.0f ? 0.0f : 1.0f / s;
        for (int64_t j = 0; j < G; ++j) {
          int q = 0;
          if (s != 0.0f) q = (int)std::min(7.0f, std::max(-8.0f, std::nearbyint(rr[g * G + j] * t)));
          put_nibble(cr, g * G + j, (uint8_t)(q & 0xF));
        }
      } else {
        const float d6 = 6.0f * alpha;
        const uint8_t sbits = f32_to_e4m3_sat(a / d6);
        ((uint8_t*)scales)[n * ng + g] = sbits;
        const float s = e4m3_to_f32(sbits);
        const float t = s == 0.0f ? 0.0f : 1.0f / (s * alpha);
        for (int64_t j = 0; j < G; ++j) {
          const uint8_t c = s == 0.0f ? 0 : f32_to_e2m1_sat(rr[g * G + j] * t);
          put_nibble(cr, g * G + j, c);
        }
      }
    }
  }
}

void orc_awq_quantize_weight(int64_t N, int64_t K, const uint16_t* w, uint8_t* codes, uint16_t* scales,
                             uint16_t* zeros) {
  const int64_t G = 64, ng = K / G;
  for (int64_t n = 0; n < N; ++n) {
    const uint16_t* wr = w + n * K;
    uint8_t* cr = codes + n * (K / 2);
    for (int64_t g = 0; g < ng; ++g) {
      float lo = 0.0f, hi = 0.0f;
      for (int64_t j = 0; j < G; ++j) {
        lo = std::min(lo, bf16_to_f32(wr[g * G + j]));
        hi = std::max(hi, bf16_to_f32(wr[g * G + j]));
      }
      const uint16_t sbits = f32_to_f16_sat((hi - lo) / 15.0f);
      const float s = f16_to_f32(sbits);
      const float t = s == 0.0f ? 0.0f : 1.0f / s;
      const float z = s == 0.0f ? 0.0f : std::min(15.0f, std::max(0.0f, std::nearbyint(-lo * t)));
      scales[n * ng + g] = sbits;
      zeros[n * ng + g] = f32_to_f16_sat(z);
      for (int64_t j = 0; j < G; ++j) {
        float q = z;
        if (s != 0.0f) q = std::min(15.0f, std::max(0.0f, std::nearbyint(bf16_to_f32(wr[g * G + j]) * t) + z));
        put_nibble(cr, g * G + j, (uint8_t)((int)q & 0xF));
      }
    }
  }
}

void orc_vec_f64_to_bf16(const double* in, uint16_t* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = f64_to_bf16(in[i]);
}

}  // extern "C"
