// Offline weight side of SVDQuant on the GPU (blog "Nunchaku 4-bit inference
// in Diffusers", "Background: SVDQuant and Nunchaku": activation outliers are
// moved into the weights, the hardest part of each weight becomes a 16-bit
// low-rank branch and the residual is quantized to 4 bits; "Nunchaku Lite",
// quantization walkthrough: the quantized checkpoint is produced offline from
// the dense weights), plus the AWQ weight quantizer:
//
//   calibrate_kernel      lambda_k = bf16(sqrt(fl32(max_m |X_mk| / max_n |W_nk|)))
//   smooth_weight_kernel  W_hat = W diag(lambda) in fp32 (exact: bf16 x bf16)
//   rank-r decomposition  randomized subspace iteration (Halko, Martinsson and
//                         Tropp, "Finding structure with randomness", 2011,
//                         Algorithm 4.4) on W_hat with a caller-supplied
//                         Gaussian test matrix, orthonormalized by CholeskyQR2,
//                         then Rayleigh-Ritz: B = Q^T W_hat, eigen-decomposition
//                         of B B^T by cyclic Jacobi rotations
//   residual_kernel       R = W_hat - (diag(lambda) L1 L2)^T with the stored bf16 factors
//   quantize_weight_kernel / awq_weight_kernel   per (row, group) 4-bit quantization
//
// Offline work, so the kernels favour plainness over speed where it does not
// matter (the small p x p steps run in one workgroup).  All sizes arrive
// validated by the C-ABI layer; every index below stays inside the buffers
// that layer checked.
#pragma clang fp contract(off)

#include <mutex>

#include "common.h"
#include "launch.h"

namespace svdq {

namespace {

// ---- calibration -----------------------------------------------------------
// One workgroup per 32 columns; 16 row slices of 16 column pairs.  The column
// maxima are exact (max is order-free), so lambda is a bit-exact function of
// the inputs.
__global__ __launch_bounds__(256) void calibrate_kernel(int Mc, int N, int K, const uint16_t* __restrict__ x,
                                                        const uint16_t* __restrict__ w, uint16_t* __restrict__ lam) {
  __shared__ float ra[16][32], rb[16][32];
  const int tid = threadIdx.x, pr = tid & 15, sl = tid >> 4;
  const int k0 = blockIdx.x * 32 + 2 * pr;  // this thread's column pair
  float a0 = 0.f, a1 = 0.f, b0 = 0.f, b1 = 0.f;
  if (k0 < K) {
    for (int m = sl; m < Mc; m += 16) {
      const u32 v = *(const u32*)(x + (size_t)m * K + k0);
      a0 = fmaxf(a0, fabsf(bf16_bits_to_f32(v & 0xFFFFu)));
      a1 = fmaxf(a1, fabsf(bf16_bits_to_f32(v >> 16)));
    }
    for (int n = sl; n < N; n += 16) {
      const u32 v = *(const u32*)(w + (size_t)n * K + k0);
      b0 = fmaxf(b0, fabsf(bf16_bits_to_f32(v & 0xFFFFu)));
      b1 = fmaxf(b1, fabsf(bf16_bits_to_f32(v >> 16)));
    }
  }
  ra[sl][2 * pr] = a0; ra[sl][2 * pr + 1] = a1;
  rb[sl][2 * pr] = b0; rb[sl][2 * pr + 1] = b1;
  __syncthreads();
  if (tid < 32 && blockIdx.x * 32 + tid < K) {
    float a = 0.f, b = 0.f;
    for (int s = 0; s < 16; ++s) {
      a = fmaxf(a, ra[s][tid]);
      b = fmaxf(b, rb[s][tid]);
    }
    const float l = (a > 0.f && b > 0.f) ? __builtin_sqrtf(a / b) : 1.0f;
    lam[blockIdx.x * 32 + tid] = (uint16_t)f32_to_bf16_bits(l);
  }
}

// ---- smoothed weight, residual ----------------------------------------------
__global__ __launch_bounds__(256) void smooth_weight_kernel(int N, int K, const uint16_t* __restrict__ w,
                                                            const uint16_t* __restrict__ lam, float* __restrict__ wh) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;  // element pair
  if (i * 2 >= (size_t)N * K) return;
  const int k = (int)((i * 2) % (size_t)K);
  const u32 v = *(const u32*)(w + 2 * i);
  const u32 l = *(const u32*)(lam + k);
  float2 o;
  o.x = bf16_bits_to_f32(v & 0xFFFFu) * bf16_bits_to_f32(l & 0xFFFFu);
  o.y = bf16_bits_to_f32(v >> 16) * bf16_bits_to_f32(l >> 16);
  *(float2*)(wh + 2 * i) = o;
}

// R[n, k] = W_hat[n, k] - sum_j L2^T[n, j] * lambda_k * L1^T[j, k] (bf16 factors)
__global__ __launch_bounds__(256) void residual_kernel(int N, int K, int r, const uint16_t* __restrict__ lam,
                                                       const uint16_t* __restrict__ l1t,
                                                       const uint16_t* __restrict__ l2t, float* __restrict__ wh) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (size_t)N * K) return;
  const int n = (int)(i / K), k = (int)(i % K);
  const float lk = bf16_bits_to_f32(lam[k]);
  float s = 0.f;
  for (int j = 0; j < r; ++j)
    s = fmaf(bf16_bits_to_f32(l2t[(size_t)n * r + j]), lk * bf16_bits_to_f32(l1t[(size_t)j * K + k]), s);
  wh[i] -= s;
}

// ---- tall-skinny products ------------------------------------------------------
// Y[n, c] = sum_k A[n, k] Z[k, c]   (A [N, K] row-major, Z [K, p], p <= 64)
// Workgroup: 32 rows x p columns; thread t owns row t / 8 (of 32) and the
// columns (t % 8) + 8 i.  K in chunks of 32 through LDS.
constexpr int TS_P = 64;
__global__ __launch_bounds__(256) void tsmm_nn_kernel(int N, int K, int p, const float* __restrict__ A,
                                                      const float* __restrict__ Z, float* __restrict__ Y) {
  __shared__ float sa[32][33];
  __shared__ float sz[32][TS_P + 1];
  const int tid = threadIdx.x, row = tid >> 3, c0 = tid & 7;
  const int n0 = blockIdx.x * 32;
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.f;
  for (int k0 = 0; k0 < K; k0 += 32) {
    for (int e = tid; e < 32 * 32; e += 256) {
      const int rr = e >> 5, kk = e & 31;
      sa[rr][kk] = (n0 + rr < N && k0 + kk < K) ? A[(size_t)(n0 + rr) * K + k0 + kk] : 0.f;
    }
    for (int e = tid; e < 32 * TS_P; e += 256) {
      const int kk = e / TS_P, cc = e % TS_P;
      sz[kk][cc] = (k0 + kk < K && cc < p) ? Z[(size_t)(k0 + kk) * p + cc] : 0.f;
    }
    __syncthreads();
#pragma unroll 4
    for (int kk = 0; kk < 32; ++kk) {
      const float a = sa[row][kk];
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = fmaf(a, sz[kk][c0 + 8 * i], acc[i]);
    }
    __syncthreads();
  }
  if (n0 + row < N) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (c0 + 8 * i < p) Y[(size_t)(n0 + row) * p + c0 + 8 * i] = acc[i];
  }
}

// Z[k, c] = sum_n A[n, k] Q[n, c]   (A^T Q; A [N, K], Q [N, p])
// Workgroup: 32 columns k x p; N in chunks of 32 through LDS (fixed order).
__global__ __launch_bounds__(256) void tsmm_tn_kernel(int N, int K, int p, const float* __restrict__ A,
                                                      const float* __restrict__ Q, float* __restrict__ Z) {
  __shared__ float sa[32][33];
  __shared__ float sq[32][TS_P + 1];
  const int tid = threadIdx.x, col = tid >> 3, c0 = tid & 7;
  const int k0 = blockIdx.x * 32;
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.f;
  for (int n0 = 0; n0 < N; n0 += 32) {
    for (int e = tid; e < 32 * 32; e += 256) {
      const int nn = e >> 5, kk = e & 31;
      sa[nn][kk] = (n0 + nn < N && k0 + kk < K) ? A[(size_t)(n0 + nn) * K + k0 + kk] : 0.f;
    }
    for (int e = tid; e < 32 * TS_P; e += 256) {
      const int nn = e / TS_P, cc = e % TS_P;
      sq[nn][cc] = (n0 + nn < N && cc < p) ? Q[(size_t)(n0 + nn) * p + cc] : 0.f;
    }
    __syncthreads();
#pragma unroll 4
    for (int nn = 0; nn < 32; ++nn) {
      const float a = sa[nn][col];
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = fmaf(a, sq[nn][c0 + 8 * i], acc[i]);
    }
    __syncthreads();
  }
  if (k0 + col < K) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (c0 + 8 * i < p) Z[(size_t)(k0 + col) * p + c0 + 8 * i] = acc[i];
  }
}

// ---- CholeskyQR ----------------------------------------------------------------
// Partial Gram matrices of row chunks: part[b][i][j] = sum_{rows of chunk b} Y[.,i] Y[.,j]
constexpr int GR_ROWS = 256;  // rows per chunk
__global__ __launch_bounds__(256) void gram_partial_kernel(int n, int p, const float* __restrict__ Y,
                                                           float* __restrict__ part) {
  __shared__ float sy[32][TS_P + 1];
  const int tid = threadIdx.x;
  const int r0 = blockIdx.x * GR_ROWS;
  // thread owns 16 entries (i, j): i = tid / 4 (0..63), j = (tid % 4) + 4 e
  const int i = tid >> 2, j0 = tid & 3;
  float acc[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) acc[e] = 0.f;
  for (int c = 0; c < GR_ROWS; c += 32) {
    for (int e = tid; e < 32 * TS_P; e += 256) {
      const int rr = e / TS_P, cc = e % TS_P;
      const int row = r0 + c + rr;
      sy[rr][cc] = (row < n && cc < p) ? Y[(size_t)row * p + cc] : 0.f;
    }
    __syncthreads();
    for (int rr = 0; rr < 32; ++rr) {
      const float yi = sy[rr][i];
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[e] = fmaf(yi, sy[rr][j0 + 4 * e], acc[e]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int e = 0; e < 16; ++e) part[((size_t)blockIdx.x * TS_P + i) * TS_P + j0 + 4 * e] = acc[e];
}

// One workgroup: sum the partial Grams in chunk order, shift (first pass only),
// Cholesky G = R^T R (R upper triangular), then Rinv = R^-1, written to rinv [p][p].
// A pivot that is not positive (possible only where the Gram matrix has a zero
// row: an all-zero input, or a column zeroed by the previous pass) marks a dead
// column: its row of R becomes e_i and its column of Rinv zero, so its basis
// vector is zero and the other columns are orthonormalized without it.
__global__ __launch_bounds__(256) void chol_inv_kernel(int p, int nparts, const float* __restrict__ part,
                                                       float shift_rel, float* __restrict__ rinv) {
  __shared__ float g[TS_P][TS_P + 1];
  __shared__ float ri[TS_P][TS_P + 1];
  __shared__ int dead[TS_P];
  __shared__ float tr;
  const int tid = threadIdx.x;
  for (int e = tid; e < p * p; e += 256) {
    const int i = e / p, j = e % p;
    float s = 0.f;
    for (int b = 0; b < nparts; ++b) s += part[((size_t)b * TS_P + i) * TS_P + j];
    g[i][j] = s;
  }
  __syncthreads();
  if (tid == 0) {
    float t = 0.f;
    for (int i = 0; i < p; ++i) t += g[i][i];
    tr = t;
  }
  __syncthreads();
  if (tid < p) g[tid][tid] += shift_rel * tr / (float)p;
  __syncthreads();
  // right-looking Cholesky on the upper triangle: row i of R
  for (int i = 0; i < p; ++i) {
    if (tid == 0) {
      const float d = g[i][i];
      dead[i] = !(d > 0.f);
      g[i][i] = dead[i] ? 1.0f : __builtin_sqrtf(d);
    }
    __syncthreads();
    const float rii = g[i][i];
    const bool di = dead[i];
    for (int j = i + 1 + tid; j < p; j += 256) g[i][j] = di ? 0.0f : g[i][j] / rii;
    __syncthreads();
    // trailing update g[a][b] -= g[i][a] g[i][b], a, b > i, b >= a
    for (int e = tid; e < (p - i - 1) * (p - i - 1); e += 256) {
      const int a = i + 1 + e / (p - i - 1), b = i + 1 + e % (p - i - 1);
      if (b >= a) g[a][b] -= g[i][a] * g[i][b];
    }
    __syncthreads();
  }
  // Rinv: upper triangular inverse by columns, thread j owns column j
  for (int e = tid; e < p * p; e += 256) ri[e / p][e % p] = 0.f;
  __syncthreads();
  if (tid < p && !dead[tid]) {
    const int j = tid;
    ri[j][j] = 1.0f / g[j][j];
    for (int i = j - 1; i >= 0; --i) {
      float s = 0.f;
      for (int k = i + 1; k <= j; ++k) s += g[i][k] * ri[k][j];
      ri[i][j] = -s / g[i][i];
    }
  }
  __syncthreads();
  for (int e = tid; e < p * p; e += 256) rinv[e] = ri[e / p][e % p];
}

// Y <- Y Rinv, one row per thread (Rinv upper triangular, in LDS)
__global__ __launch_bounds__(256) void apply_rinv_kernel(int n, int p, const float* __restrict__ rinv,
                                                         float* __restrict__ Y) {
  __shared__ float ri[TS_P * TS_P];
  for (int e = threadIdx.x; e < p * p; e += 256) ri[e] = rinv[e];
  __syncthreads();
  const int row = blockIdx.x * 256 + threadIdx.x;
  if (row >= n) return;
  float y[TS_P];
  for (int c = 0; c < p; ++c) y[c] = Y[(size_t)row * p + c];
  for (int c = p - 1; c >= 0; --c) {
    float s = 0.f;
    for (int i = 0; i <= c; ++i) s = fmaf(y[i], ri[i * p + c], s);
    Y[(size_t)row * p + c] = s;
  }
}

// ---- Rayleigh-Ritz: eigen-decomposition of C = Zb^T Zb (p x p) ---------------
// One workgroup: cyclic Jacobi sweeps on C in LDS, eigenvectors accumulated in
// E; then eigenpairs sorted by decreasing eigenvalue.  out: evals [p], evecs [p][p]
// (column j = eigenvector j).
__global__ __launch_bounds__(256) void jacobi_eig_kernel(int p, int nparts, const float* __restrict__ part,
                                                         int sweeps, float* __restrict__ evals,
                                                         float* __restrict__ evecs) {
  __shared__ float c[TS_P][TS_P + 1];
  __shared__ float e[TS_P][TS_P + 1];
  __shared__ float cs[2];
  const int tid = threadIdx.x;
  for (int t = tid; t < p * p; t += 256) {
    const int i = t / p, j = t % p;
    float s = 0.f;
    for (int b = 0; b < nparts; ++b) s += part[((size_t)b * TS_P + i) * TS_P + j];
    c[i][j] = s;
    e[i][j] = i == j ? 1.f : 0.f;
  }
  __syncthreads();
  for (int sw = 0; sw < sweeps; ++sw) {
    for (int a = 0; a < p - 1; ++a)
      for (int b = a + 1; b < p; ++b) {
        if (tid == 0) {
          const float apq = c[a][b];
          float co = 1.f, si = 0.f;
          if (fabsf(apq) > 1e-30f) {
            const float th = (c[b][b] - c[a][a]) / (2.f * apq);
            const float t = (th >= 0.f ? 1.f : -1.f) / (fabsf(th) + __builtin_sqrtf(th * th + 1.f));
            co = 1.f / __builtin_sqrtf(t * t + 1.f);
            si = t * co;
          }
          cs[0] = co;
          cs[1] = si;
        }
        __syncthreads();
        const float co = cs[0], si = cs[1];
        if (si != 0.f) {
          // C <- J^T C J: rows a, b then columns a, b
          if (tid < p) {
            const float ca = c[a][tid], cb = c[b][tid];
            c[a][tid] = co * ca - si * cb;
            c[b][tid] = si * ca + co * cb;
          }
          __syncthreads();
          if (tid < p) {
            const float ca = c[tid][a], cb = c[tid][b];
            c[tid][a] = co * ca - si * cb;
            c[tid][b] = si * ca + co * cb;
            const float ea = e[tid][a], eb = e[tid][b];
            e[tid][a] = co * ea - si * eb;
            e[tid][b] = si * ea + co * eb;
          }
        }
        __syncthreads();
      }
  }
  // sort by decreasing eigenvalue (selection order computed by one thread)
  __shared__ int order[TS_P];
  if (tid == 0) {
    bool used[TS_P];
    for (int i = 0; i < p; ++i) used[i] = false;
    for (int i = 0; i < p; ++i) {
      int best = -1;
      for (int j = 0; j < p; ++j)
        if (!used[j] && (best < 0 || c[j][j] > c[best][best])) best = j;
      used[best] = true;
      order[i] = best;
    }
  }
  __syncthreads();
  if (tid < p) evals[tid] = c[order[tid]][order[tid]];
  for (int t = tid; t < p * p; t += 256) {
    const int i = t / p, j = t % p;
    evecs[i * p + j] = e[i][order[j]];
  }
}

// Factors of the layer from the Ritz vectors (first r):
//   l2t[n, j] = bf16(sqrt(s_j) (Q E)[n, j]),  l1t[j, k] = bf16((1/lambda_k) (Zb E)[k, j] / sqrt(s_j))
// with s_j = sqrt(eval_j) the singular values.  One thread per (row, j).
__global__ __launch_bounds__(256) void factors_kernel(int n_rows, int p, int r, int is_l1, const float* __restrict__ M,
                                                      const float* __restrict__ evals, const float* __restrict__ evecs,
                                                      const uint16_t* __restrict__ lam, int K,
                                                      uint16_t* __restrict__ out) {
  const size_t t = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= (size_t)n_rows * r) return;
  const int row = (int)(t / r), j = (int)(t % r);
  float s = 0.f;
  for (int i = 0; i < p; ++i) s = fmaf(M[(size_t)row * p + i], evecs[i * p + j], s);
  const float sv = __builtin_sqrtf(fmaxf(evals[j], 0.f));  // singular value
  const float rs = __builtin_sqrtf(sv);
  if (is_l1) {
    const float v = rs > 0.f ? s / rs : 0.f;   // (Zb E)/s_j * sqrt(s_j)
    const float l = lam ? bf16_bits_to_f32(lam[row]) : 1.0f;
    out[(size_t)j * K + row] = (uint16_t)f32_to_bf16_bits(v / l);
  } else {
    out[(size_t)row * r + j] = (uint16_t)f32_to_bf16_bits(s * rs);
  }
}

// ---- 4-bit weight quantizers --------------------------------------------------
// One thread per (row, group): the activation quantizer's steps on an fp32
// input (int4 group 64 / nvfp4 group 16).
template <int PREC>
__global__ __launch_bounds__(256) void quantize_weight_kernel(int N, int K, const float* __restrict__ r, float alpha,
                                                              uint8_t* __restrict__ codes, void* __restrict__ scales) {
  constexpr int G = PREC == 0 ? 64 : 16;
  const int ng = K / G;
  const size_t t = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= (size_t)N * ng) return;
  const int n = (int)(t / ng), g = (int)(t % ng);
  const float* src = r + (size_t)n * K + g * G;
  float v[G];
  float a = 0.f;
#pragma unroll
  for (int i = 0; i < G; i += 4) {
    const float4 q = *(const float4*)(src + i);
    v[i] = q.x; v[i + 1] = q.y; v[i + 2] = q.z; v[i + 3] = q.w;
    a = fmaxf(a, fmaxf(fmaxf(fabsf(q.x), fabsf(q.y)), fmaxf(fabsf(q.z), fabsf(q.w))));
  }
  uint8_t* dst = codes + (size_t)n * (K / 2) + g * (G / 2);
  if constexpr (PREC == 0) {
    const u32 sbits = f32_to_f16_sat_bits(a / 7.0f);
    ((uint16_t*)scales)[(size_t)n * ng + g] = (uint16_t)sbits;
    const float s = f16_bits_to_f32(sbits);
    const float tt = s == 0.f ? 0.f : 1.0f / s;
#pragma unroll
    for (int i = 0; i < G; i += 8) {
      u32 w = 0u;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float q = __builtin_rintf(v[i + e] * tt);
        q = fminf(fmaxf(q, -8.0f), 7.0f);
        w |= ((u32)(int)q & 0xFu) << (4 * e);
      }
      *(u32*)(dst + i / 2) = w;
    }
  } else {
    const u32 sbits = f32_to_e4m3_sat_pos(a / (6.0f * alpha));
    ((uint8_t*)scales)[(size_t)n * ng + g] = (uint8_t)sbits;
    const float s = e4m3_to_f32(sbits);
    float tt = 0.f;
    if (s != 0.f) {
      const float sa = s * alpha;
      tt = 1.0f / sa;
    }
#pragma unroll
    for (int i = 0; i < G; i += 8) *(u32*)(dst + i / 2) = s == 0.f ? 0u : e2m1_codes8(v + i, tt);
  }
}

// AWQ: min-max over a range containing 0, per (row, 64-group)
__global__ __launch_bounds__(256) void awq_weight_kernel(int N, int K, const uint16_t* __restrict__ w,
                                                         uint8_t* __restrict__ codes, uint16_t* __restrict__ scales,
                                                         uint16_t* __restrict__ zeros) {
  const int ng = K / 64;
  const size_t t = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= (size_t)N * ng) return;
  const int n = (int)(t / ng), g = (int)(t % ng);
  const uint16_t* src = w + (size_t)n * K + g * 64;
  float v[64];
  float lo = 0.f, hi = 0.f;
#pragma unroll
  for (int i = 0; i < 64; i += 8) {
    const uint4 q = *(const uint4*)(src + i);
    const u32 wd[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[i + 2 * e] = bf16_bits_to_f32(wd[e] & 0xFFFFu);
      v[i + 2 * e + 1] = bf16_bits_to_f32(wd[e] >> 16);
    }
  }
#pragma unroll
  for (int i = 0; i < 64; ++i) {
    lo = fminf(lo, v[i]);
    hi = fmaxf(hi, v[i]);
  }
  const u32 sbits = f32_to_f16_sat_bits((hi - lo) / 15.0f);
  const float s = f16_bits_to_f32(sbits);
  const float tt = s == 0.f ? 0.f : 1.0f / s;
  const float z = s == 0.f ? 0.f : fminf(15.f, fmaxf(0.f, __builtin_rintf(-lo * tt)));
  scales[(size_t)n * ng + g] = (uint16_t)sbits;
  zeros[(size_t)n * ng + g] = (uint16_t)f32_to_f16_sat_bits(z);
  uint8_t* dst = codes + (size_t)n * (K / 2) + g * 32;
#pragma unroll
  for (int i = 0; i < 64; i += 8) {
    u32 wd = 0u;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float q = s == 0.f ? z : fminf(15.f, fmaxf(0.f, __builtin_rintf(v[i + e] * tt) + z));
      wd |= ((u32)(int)q & 0xFu) << (4 * e);
    }
    *(u32*)(dst + i / 2) = wd;
  }
}

inline unsigned blocks_for(size_t n, unsigned per) { return (unsigned)((n + per - 1) / per); }

}  // namespace

// Fixed workspace of the allocation-free decomposition entry point: one copy
// per GPU, held until the process ends.  Host code never uses this name as an
// address (on the host it is only a stand-in for the symbol); the device
// address comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

hipError_t noalloc_scratch(void** ptr) {
  static std::mutex mu;
  static void* addr[64] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

size_t lowrank_workspace_bytes(int64_t N, int64_t K, int p) {
  const int64_t rows = N > K ? N : K;
  const size_t parts = (size_t)((rows + GR_ROWS - 1) / GR_ROWS);
  return sizeof(float) * ((size_t)N * p            // Y / Q
                          + (size_t)K * p          // Z
                          + parts * TS_P * TS_P    // partial Grams
                          + TS_P * TS_P            // Rinv
                          + TS_P + TS_P * TS_P);   // evals, evecs
}

hipError_t launch_calibrate(int64_t Mc, int64_t N, int64_t K, const void* x, const void* w, void* lam, hipStream_t st) {
  hipLaunchKernelGGL(calibrate_kernel, dim3(blocks_for(K, 32)), dim3(256), 0, st, (int)Mc, (int)N, (int)K,
                     (const uint16_t*)x, (const uint16_t*)w, (uint16_t*)lam);
  return hipGetLastError();
}

// Orthonormalize Y [n, p] in place (CholeskyQR2; a small diagonal shift on the
// first pass keeps the Gram matrix positive definite in fp32).
static void orth(int n, int p, float* Y, float* part, float* rinv, hipStream_t st) {
  const int nparts = (n + GR_ROWS - 1) / GR_ROWS;
  for (int pass = 0; pass < 2; ++pass) {
    hipLaunchKernelGGL(gram_partial_kernel, dim3(nparts), dim3(256), 0, st, n, p, (const float*)Y, part);
    hipLaunchKernelGGL(chol_inv_kernel, dim3(1), dim3(256), 0, st, p, nparts, (const float*)part,
                       pass == 0 ? 1e-6f : 0.0f, rinv);
    hipLaunchKernelGGL(apply_rinv_kernel, dim3(blocks_for(n, 256)), dim3(256), 0, st, n, p, (const float*)rinv, Y);
  }
}

hipError_t launch_lowrank(const LowrankArgs& a, hipStream_t st) {
  const int N = (int)a.N, K = (int)a.K, p = a.p, r = a.rank;
  float* ws = (float*)a.work;
  float* Y = ws;                              // [N, p]
  float* Z = Y + (size_t)N * p;               // [K, p]
  const int64_t rows = a.N > a.K ? a.N : a.K;
  const size_t parts = (size_t)((rows + GR_ROWS - 1) / GR_ROWS);
  float* part = Z + (size_t)K * p;            // [parts][64][64]
  float* rinv = part + parts * TS_P * TS_P;   // [64][64]
  float* evals = rinv + TS_P * TS_P;          // [64]
  float* evecs = evals + TS_P;                // [64][64]
  float* wh = a.residual;
  hipLaunchKernelGGL(smooth_weight_kernel, dim3(blocks_for((size_t)N * K / 2, 256)), dim3(256), 0, st, N, K,
                     (const uint16_t*)a.w, (const uint16_t*)a.lam, wh);
  const hipError_t e = hipMemcpyAsync(Z, a.omega, sizeof(float) * (size_t)K * p, hipMemcpyDeviceToDevice, st);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(tsmm_nn_kernel, dim3(blocks_for(N, 32)), dim3(256), 0, st, N, K, p, (const float*)wh,
                     (const float*)Z, Y);
  orth(N, p, Y, part, rinv, st);
  for (int it = 0; it < a.iters; ++it) {
    hipLaunchKernelGGL(tsmm_tn_kernel, dim3(blocks_for(K, 32)), dim3(256), 0, st, N, K, p, (const float*)wh,
                       (const float*)Y, Z);
    orth(K, p, Z, part, rinv, st);
    hipLaunchKernelGGL(tsmm_nn_kernel, dim3(blocks_for(N, 32)), dim3(256), 0, st, N, K, p, (const float*)wh,
                       (const float*)Z, Y);
    orth(N, p, Y, part, rinv, st);
  }
  // Rayleigh-Ritz: Zb = W_hat^T Q [K, p]; C = Zb^T Zb; C = E diag(ev) E^T
  hipLaunchKernelGGL(tsmm_tn_kernel, dim3(blocks_for(K, 32)), dim3(256), 0, st, N, K, p, (const float*)wh,
                     (const float*)Y, Z);
  const int kparts = (K + GR_ROWS - 1) / GR_ROWS;
  hipLaunchKernelGGL(gram_partial_kernel, dim3(kparts), dim3(256), 0, st, K, p, (const float*)Z, part);
  hipLaunchKernelGGL(jacobi_eig_kernel, dim3(1), dim3(256), 0, st, p, kparts, (const float*)part, 12, evals, evecs);
  hipLaunchKernelGGL(factors_kernel, dim3(blocks_for((size_t)N * r, 256)), dim3(256), 0, st, N, p, r, 0,
                     (const float*)Y, (const float*)evals, (const float*)evecs, (const uint16_t*)nullptr, K,
                     (uint16_t*)a.l2t);
  hipLaunchKernelGGL(factors_kernel, dim3(blocks_for((size_t)K * r, 256)), dim3(256), 0, st, K, p, r, 1,
                     (const float*)Z, (const float*)evals, (const float*)evecs, (const uint16_t*)a.lam, K,
                     (uint16_t*)a.l1t);
  hipLaunchKernelGGL(residual_kernel, dim3(blocks_for((size_t)N * K, 256)), dim3(256), 0, st, N, K, r,
                     (const uint16_t*)a.lam, (const uint16_t*)a.l1t, (const uint16_t*)a.l2t, wh);
  return hipGetLastError();
}

hipError_t launch_quantize_weight(int precision, int64_t N, int64_t K, const float* r, float alpha, void* codes,
                                  void* scales, hipStream_t st) {
  const int G = precision == 0 ? 64 : 16;
  const unsigned nb = blocks_for((size_t)N * (K / G), 256);
  if (precision == 0)
    hipLaunchKernelGGL(quantize_weight_kernel<0>, dim3(nb), dim3(256), 0, st, (int)N, (int)K, r, alpha,
                       (uint8_t*)codes, scales);
  else
    hipLaunchKernelGGL(quantize_weight_kernel<1>, dim3(nb), dim3(256), 0, st, (int)N, (int)K, r, alpha,
                       (uint8_t*)codes, scales);
  return hipGetLastError();
}

hipError_t launch_awq_quantize(int64_t N, int64_t K, const void* w, void* codes, void* scales, void* zeros,
                               hipStream_t st) {
  hipLaunchKernelGGL(awq_weight_kernel, dim3(blocks_for((size_t)N * (K / 64), 256)), dim3(256), 0, st, (int)N,
                     (int)K, (const uint16_t*)w, (uint8_t*)codes, (uint16_t*)scales, (uint16_t*)zeros);
  return hipGetLastError();
}

}  // namespace svdq
