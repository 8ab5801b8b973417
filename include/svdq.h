/*
 * svdq.h -- C ABI of libsvdq.so: the SVDQuant W4A4 linear layer and the AWQ
 * W4A16 weight-only linear, as hand-written HIP kernels for AMD Instinct
 * MI355X (gfx950).
 *
 * What the layer computes (sources: the "Nunchaku Lite" Diffusers docs and the
 * blog "Nunchaku 4-bit inference in Diffusers"):
 *   Y = Q(X / lambda) . Q(W_res)^T  with per-group dequantization
 *     + (X . L1) . L2                16-bit low-rank branch
 *     + bias
 *   - smoothing moves activation outliers into the weights; a low-rank branch
 *     carries the hardest part of each weight; the residual runs as 4-bit
 *     weights x 4-bit activations (blog, "Background: SVDQuant and Nunchaku");
 *   - the low-rank down-projection X.L1 is computed by the activation quantizer
 *     and the up-projection (X.L1).L2 inside the 4-bit GEMM, so the 16-bit
 *     branch adds no extra pass over X or Y (same section);
 *   - precisions: svdq_w4a4 int4 with group 64, svdq_w4a4 nvfp4 with group 16,
 *     awq_w4a16 int4 weight-only with group 64 ("Nunchaku Lite", table in
 *     "Supported quantization types"); the layer's float buffers are bfloat16
 *     ("NunchakuLiteQuantizationConfig", compute_dtype);
 *   - an unsupported GPU is reported as an error, never as wrong output (blog,
 *     "Hardware support").
 *
 * Conventions shared by every entry point
 *   - All buffers are caller-owned DEVICE pointers, contiguous, row-major,
 *     16-byte aligned.  The library allocates nothing and keeps no state apart
 *     from a per-device architecture check.
 *   - bf16 / fp16 values are IEEE bit patterns in uint16; E4M3 values are OCP
 *     E4M3 "FN" bytes; 4-bit codes are packed two per byte, even channel k in
 *     the low nibble.  int4 codes are two's complement in [-8, 7]; NVFP4 codes
 *     are E2M1 (sign in bit 3); AWQ codes are unsigned 0..15.
 *   - Weights follow the nn.Linear layout: W codes [N, K/2], L1 given as
 *     l1t = L1^T [rank, K], L2 given as l2t = L2^T [N, rank].
 *   - `stream` is a hipStream_t (NULL = the default stream).  Every call only
 *     enqueues work on it and returns; nothing synchronizes.  A device fault
 *     of an earlier launch is reported by the next call as SVDQ_ERR_DEVICE.
 *   - Every argument is checked before anything is launched; on a non-OK
 *     status nothing was enqueued and svdq_last_error() describes the cause.
 *   - M == 0 is a valid empty call: nothing is launched and the buffers whose
 *     size is proportional to M may be NULL.
 */
#ifndef SVDQ_H_
#define SVDQ_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SVDQ_OK = 0,
  SVDQ_ERR_INVALID_ARG = 1,  /* NULL required pointer, negative or inconsistent size */
  SVDQ_ERR_UNSUPPORTED = 2,  /* not gfx950, precision/group/rank outside the table, shape limits */
  SVDQ_ERR_ALIGNMENT = 3,    /* a pointer is not 16-byte aligned */
  SVDQ_ERR_DEVICE = 4        /* a HIP runtime error (launch failure or an earlier fault) */
} svdq_status;

typedef enum { SVDQ_INT4 = 0, SVDQ_NVFP4 = 1 } svdq_precision;

/*
 * svdq_quantize_act -- smoothing, 4-bit activation quantization and the fused
 * low-rank down-projection, reading X once (blog, "Background: SVDQuant and
 * Nunchaku"; precisions from "Supported quantization types").
 *
 * For every row m and group g of `group_size` channels:
 *   xh_k = fl32(x_k * fl32(1 / lambda_k))                  (smoothing)
 *   int4 (group 64):  s = fp16_sat(fl32(max|xh| / 7)),
 *                     q_k = clamp(rne(fl32(xh_k * fl32(1/s))), -8, 7), 0 if s == 0
 *   nvfp4 (group 16): s = e4m3_sat(fl32(max|xh| / fl32(6 * alpha))),
 *                     c_k = e2m1_sat(fl32(xh_k * fl32(1 / fl32(s * alpha)))), 0 if s == 0
 *   xl1[m, j] = sum_k x[m, k] * L1[k, j]   (raw X, fp32 accumulation)
 *
 *   precision   SVDQ_INT4 (group_size must be 64) or SVDQ_NVFP4 (16)
 *   rank        0, 16, 32, ..., 128; 0 disables the low-rank branch
 *   M, K        rows and channels; K % 64 == 0, K <= 32768, M*K < 2^30,
 *               M*rank*4 < 2^31 (32-bit byte offsets into xl1)
 *   x           bf16 [M, K]; +-inf quantizes to the saturated code of its sign
 *               (int4 -8 / 7, nvfp4 -6 / 6) and counts as the group's maximum;
 *               codes and scales of a group holding a NaN are unspecified
 *   smooth      bf16 [K] smoothing factors lambda (finite, > 0), or NULL for 1
 *   l1t         bf16 [rank, K] (L1 transposed); NULL iff rank == 0
 *   act_global_scale  NVFP4 per-tensor scale alpha > 0 (static); ignored for int4
 *   act_codes   out u8 [M, K/2]
 *   act_scales  out int4: fp16 [M, K/64]; nvfp4: E4M3 u8 [M, K/16]
 *   xl1         out fp32 [M, rank]; NULL iff rank == 0
 */
svdq_status svdq_quantize_act(int precision, int group_size, int rank, int64_t M, int64_t K,
                              const void* x, const void* smooth, const void* l1t,
                              float act_global_scale, void* act_codes, void* act_scales,
                              float* xl1, void* stream);

/*
 * svdq_quantize_act_ws -- svdq_quantize_act with the workspace of
 * svdq_w4a4_gemm_ws (SVDQ_GEMM_WORK_BYTES, declared below): the same
 * smoothing, quantization and fused down-projection (blog, "Background:
 * SVDQuant and Nunchaku"), with the work of a call that has fewer 32-row
 * blocks than the device has CUs spread evenly over all of them: the grid of
 * (32-row block, 64-channel step) pairs is cut into equal contiguous ranges,
 * one per workgroup, so a block can be shared by two or more workgroups.
 * Codes and scales are those of svdq_quantize_act bit for bit.  The rows of
 * a shared block get XL1 as the sum of the pieces' fp32 partial tiles, met
 * in `work` and added in a fixed order by the last piece to finish, so their
 * XL1 can differ from svdq_quantize_act's in the last bits (the same bits
 * from call to call).  The split applies to ranks 16 and 32 where K is a
 * whole number of 256-channel rounds (of 2048-channel chunks for K > 4096)
 * and it shortens each workgroup's share by at least 2048 channels of a
 * block (fewer blocks than CUs); elsewhere the call is svdq_quantize_act.
 *
 *   work        NULL (then exactly svdq_quantize_act; work_bytes must be 0), or
 *               the workspace of svdq_w4a4_gemm_ws: at least
 *               SVDQ_GEMM_WORK_BYTES bytes, 16-byte aligned, not overlapping
 *               an input or output, zero-filled before its first use.  A call
 *               leaves its counter words zero again (they sit apart from the
 *               GEMM's), so one workspace serves the quantizer and the GEMMs of
 *               one stream; calls that may run at the same time (other streams)
 *               need workspaces of their own.
 *   work_bytes  its size in bytes
 *   the other arguments, limits and errors as for svdq_quantize_act
 */
svdq_status svdq_quantize_act_ws(int precision, int group_size, int rank, int64_t M, int64_t K,
                                 const void* x, const void* smooth, const void* l1t,
                                 float act_global_scale, void* act_codes, void* act_scales,
                                 float* xl1, void* work, int64_t work_bytes, void* stream);

/*
 * svdq_w4a4_gemm -- the 4-bit GEMM with per-group dequantization and the
 * low-rank up-projection and bias fused into its epilogue (blog, "Background:
 * SVDQuant and Nunchaku"):
 *   int4:  y[m,n] = sum_g sa[m,g] * sw[n,g] * P[m,n,g]
 *   nvfp4: y[m,n] = alpha_a * alpha_w * sum_g sa[m,g] * sw[n,g] * P[m,n,g]
 *          + sum_j xl1[m,j] * L2[j,n] + bias[n];   Y = bf16(y)
 * where P[m,n,g] = sum over the group's channels of act code x weight code.
 *
 *   precision, group_size   as for svdq_quantize_act
 *   rank        0, 16, ..., 128
 *   M, N, K     M >= 0; N % 128 == 0; K % 64 == 0, K <= 32768 (the largest K
 *               parity-tested); M*K, N*K, M*N <= 2^31; M*rank*4 and N*rank*2
 *               below 2^31 (32-bit byte offsets into xl1 and l2t)
 *   act_codes, act_scales   as written by svdq_quantize_act
 *   act_global_scale, w_global_scale   NVFP4 alpha_a, alpha_w (each finite and
 *               > 0, and their fp32 product a finite normal float: the epilogue
 *               applies that one factor); ignored for int4
 *   w_codes     u8 [N, K/2] (same nibble order and encoding as act_codes)
 *   w_scales    int4: fp16 [N, K/64]; nvfp4: E4M3 u8 [N, K/16]
 *   xl1         fp32 [M, rank]; NULL iff rank == 0
 *   l2t         bf16 [N, rank] (L2 transposed); NULL iff rank == 0
 *   bias        bf16 [N] or NULL
 *   y           out bf16 [M, N]; must not overlap any input
 */
svdq_status svdq_w4a4_gemm(int precision, int group_size, int rank, int64_t M, int64_t N,
                           int64_t K, const void* act_codes, const void* act_scales,
                           float act_global_scale, const void* w_codes, const void* w_scales,
                           float w_global_scale, const float* xl1, const void* l2t,
                           const void* bias, void* y, void* stream);

/*
 * svdq_w4a4_gemm_ws -- svdq_w4a4_gemm with a caller-owned workspace: the same
 * product (blog, "Background: SVDQuant and Nunchaku"), where the kernel may
 * run the tiles of its grid's last partial round as K slices spread over the
 * CUs (int4 and nvfp4; nvfp4 slices are whole 1024-channel blocks of K).
 * The slices' fp32 partial accumulators meet in `work`, and the last slice of
 * a tile to finish adds them up in slice order and writes the tile.
 * Those tiles' fp32 sums are then formed in another order than
 * svdq_w4a4_gemm's, so their Y can differ from it in the last bit (the same
 * bits from call to call).
 *
 *   work        NULL (then exactly svdq_w4a4_gemm; work_bytes must be 0), or
 *               device memory of at least SVDQ_GEMM_WORK_BYTES bytes, 16-byte
 *               aligned, not overlapping y or an input, zero-filled before
 *               its first use.  A call leaves its counter words zero again (the
 *               rest is scratch), so the same workspace serves every later
 *               call on the same stream; calls that may run at the same time
 *               (other streams) need workspaces of their own.
 *   work_bytes  its size in bytes
 *   the other arguments, limits and errors as for svdq_w4a4_gemm
 */
#define SVDQ_GEMM_WORK_BYTES ((int64_t)16 * 1024 * 1024 + 4096)
svdq_status svdq_w4a4_gemm_ws(int precision, int group_size, int rank, int64_t M, int64_t N,
                              int64_t K, const void* act_codes, const void* act_scales,
                              float act_global_scale, const void* w_codes, const void* w_scales,
                              float w_global_scale, const float* xl1, const void* l2t,
                              const void* bias, void* y, void* work, int64_t work_bytes, void* stream);

/*
 * svdq_w4a4_gemm_qkv_norm_rope -- the fused attention projection: the 4-bit
 * GEMM of the grouped Q/K/V weights with the per-head RMSNorm of Q and K and
 * the rotary embedding applied to its fp32 result inside the epilogue, so Y
 * is written once ("Nunchaku Lite", "Fused kernels"; blog, "Quantizing models
 * with structural rewrites": Q, K and V weights concatenated along the output
 * dimension in that order, one operator for projection, norms and rotary
 * embedding):
 *   y   = the svdq_w4a4_gemm result (bias included) before rounding, with
 *         columns [Q | K | V], each heads * head_dim wide, head h of Q at
 *         columns h*head_dim .. +head_dim-1 (K likewise after Q)
 *   for every token m and every head of Q (weights w = norm_q) and of K (norm_k):
 *     u_d = y_d * w_d / sqrt(mean_d(y_d^2) + eps)            d = 0 .. head_dim-1
 *     (u_2p, u_2p+1) <- (u_2p*c - u_2p+1*s, u_2p*s + u_2p+1*c),
 *     (c, s) = rope[m mod rope_rows][p]
 *   V columns are y unchanged; Y = bf16 of the result.
 *
 *   heads, head_dim   head_dim 64 or 128; N = 3 * heads * head_dim must be a
 *                     multiple of 128 (N is implied, not passed)
 *   norm_q, norm_k    bf16 [head_dim]; required when M > 0
 *   eps               finite, >= 0
 *   rope              fp32 [rope_rows, head_dim/2, 2] (cos, sin) pairs, or NULL
 *                     for no rotary embedding; token rows are batch-major, so
 *                     rope_rows is the sequence length (>= 1 when rope is given)
 *   y                 out bf16 [M, N]; must not overlap any input
 *   other arguments and limits as for svdq_w4a4_gemm.
 */
svdq_status svdq_w4a4_gemm_qkv_norm_rope(int precision, int group_size, int rank, int64_t M,
                                         int heads, int head_dim, int64_t K, const void* act_codes,
                                         const void* act_scales, float act_global_scale,
                                         const void* w_codes, const void* w_scales,
                                         float w_global_scale, const float* xl1, const void* l2t,
                                         const void* bias, const void* norm_q, const void* norm_k,
                                         float eps, const float* rope, int64_t rope_rows, void* y,
                                         void* stream);

/*
 * svdq_w4a4_gemm_qkv_norm_rope_ws -- svdq_w4a4_gemm_qkv_norm_rope with the
 * workspace of svdq_w4a4_gemm_ws: the grid's last partial round of tiles may
 * run as K slices, and the last slice of a tile runs the norm and rotary
 * epilogue on the summed tile.  work, work_bytes as for svdq_w4a4_gemm_ws;
 * everything else as for svdq_w4a4_gemm_qkv_norm_rope.
 */
svdq_status svdq_w4a4_gemm_qkv_norm_rope_ws(int precision, int group_size, int rank, int64_t M,
                                            int heads, int head_dim, int64_t K, const void* act_codes,
                                            const void* act_scales, float act_global_scale,
                                            const void* w_codes, const void* w_scales,
                                            float w_global_scale, const float* xl1, const void* l2t,
                                            const void* bias, const void* norm_q, const void* norm_k,
                                            float eps, const float* rope, int64_t rope_rows, void* y,
                                            void* work, int64_t work_bytes, void* stream);

/*
 * svdq_w4a4_gemm_gelu_quant -- the fused MLP up-projection: the W4A4 GEMM of
 * the up projection, GELU, and the down projection's activation quantization
 * and low-rank input, all in the GEMM's epilogue, so the [M, N] hidden
 * activation is never written ("Nunchaku Lite", "Fused kernels": the GELU MLP
 * fusion of the original engine; blog, "Background: SVDQuant and Nunchaku"
 * for the quantizer and the low-rank branch):
 *   y  = the svdq_w4a4_gemm result (bias included) before rounding, [M, N]
 *   h  = bf16(GELU(y)),  GELU(y) = y * Phi(y) (erf form; the kernel evaluates
 *        Phi with a rational approximation of absolute error below 1e-7)
 *   codes_out, scales_out = svdq_quantize_act(precision, group_size) of h with
 *        smoothing smooth_out and, for nvfp4, global scale out_global_scale
 *        (the same decisions, taken on the kernel's h)
 *   xl1_out = h . L1_out  (fp32, [M, rank_out]; the column tiles' shares are
 *        summed with fp32 atomics, so the summation order, and the last bits,
 *        can differ between calls)
 * The outputs feed svdq_w4a4_gemm of the down projection (K = N, act_global_scale
 * = out_global_scale).  Both projections take the same precision.
 *
 *   precision   SVDQ_INT4 (group_size 64) or SVDQ_NVFP4 (group_size 16)
 *   rank, M, N, K, act_*, w_*, xl1, l2t, bias   as for svdq_w4a4_gemm
 *   smooth_out  bf16 [N] smoothing factors of the down projection, or NULL for 1
 *   l1t_out     bf16 [rank_out, N] (L1 of the down projection, transposed);
 *               NULL iff rank_out == 0
 *   rank_out    0, 16, ..., 128; M*rank_out*4 < 2^31
 *   out_global_scale  nvfp4: the down projection's activation global scale
 *               (finite, > 0, fl32(6 * it) normal); ignored for int4
 *   codes_out   out u8 [M, N/2]; scales_out out fp16 [M, N/64] (int4) or
 *               E4M3 u8 [M, N/16] (nvfp4)
 *   xl1_out     out fp32 [M, rank_out] (NULL iff rank_out == 0)
 * No output may overlap an input or another output.
 */
svdq_status svdq_w4a4_gemm_gelu_quant(int precision, int group_size, int rank, int64_t M, int64_t N,
                                     int64_t K, const void* act_codes, const void* act_scales,
                                     float act_global_scale, const void* w_codes, const void* w_scales,
                                     float w_global_scale, const float* xl1, const void* l2t,
                                     const void* bias, const void* smooth_out, const void* l1t_out,
                                     int rank_out, float out_global_scale, void* codes_out,
                                     void* scales_out, float* xl1_out, void* stream);

/*
 * awq_w4a16_gemv -- AWQ-style int4 weight-only linear for memory-bound
 * modulation projections ("Supported quantization types": awq_w4a16, int4,
 * group 64; blog, "Introducing Nunchaku Lite"):
 *   y[m,n] = sum_g sum_{k in g} x[m,k] * (q[n,k] - z[n,g]) * s[n,g] + bias[n]
 *
 *   group_size  64
 *   M, N, K     0 <= M <= 64; N % 64 == 0; K % 64 == 0; M*K < 2^30
 *   x           bf16 [M, K]
 *   w_codes     u8 [N, K/2], unsigned codes 0..15
 *   w_scales    fp16 [N, K/64]
 *   w_zeros     fp16 [N, K/64] (zero-points, in code units)
 *   bias        bf16 [N] or NULL
 *   y           out bf16 [M, N]
 */
svdq_status awq_w4a16_gemv(int group_size, int64_t M, int64_t N, int64_t K, const void* x,
                           const void* w_codes, const void* w_scales, const void* w_zeros,
                           const void* bias, void* y, void* stream);

/*
 * svdq_quantize_act_awq_gemv -- svdq_quantize_act and an independent
 * awq_w4a16_gemv in one launch where the shapes allow it: the smoothing,
 * quantization and fused down-projection of one layer's activations (blog,
 * "Background: SVDQuant and Nunchaku") beside a memory-bound AWQ projection
 * (blog, "Introducing Nunchaku Lite": the modulation projections are
 * weight-only), for a step that has both at hand, e.g. a DiT block's
 * attention input and a later block's modulation, which depends only on the
 * timestep embedding.  The quantizer of a DiT-sized call holds a part of the
 * CUs (one 32-row workgroup each); the GEMV's workgroups run on the others
 * meanwhile.  Every output is bit-identical to the two separate calls.
 *
 *   the first twelve arguments   as for svdq_quantize_act (no workspace)
 *   awq_group_size .. y          as for awq_w4a16_gemv (awq_M, awq_N, awq_K,
 *                                awq_x are its M, N, K, x)
 * The AWQ output must not overlap any quantizer buffer, nor a quantizer
 * output any AWQ input.  Either job may be empty (M == 0 / awq_M == 0).
 * One launch when the quantizer runs its LDS-staged kernel unsplit (ranks 16
 * and 32, more 16-row blocks than CUs, K <= 4096) and the GEMV its small-M
 * kernel (awq_M <= 4, awq_K % 512 == 0, awq_K <= 8192, awq_N % 32 == 0);
 * otherwise the two launches, quantizer first, on the same stream.  Limits
 * and errors as for the two calls; nothing is enqueued unless both
 * validate.
 */
svdq_status svdq_quantize_act_awq_gemv(int precision, int group_size, int rank, int64_t M, int64_t K,
                                       const void* x, const void* smooth, const void* l1t,
                                       float act_global_scale, void* act_codes, void* act_scales, float* xl1,
                                       int awq_group_size, int64_t awq_M, int64_t awq_N, int64_t awq_K,
                                       const void* awq_x, const void* w_codes, const void* w_scales,
                                       const void* w_zeros, const void* bias, void* y, void* stream);

/* ---------------------------------------------------------------------------
 * Offline weight side (blog "Nunchaku 4-bit inference in Diffusers",
 * "Background: SVDQuant and Nunchaku": activation outliers move into the
 * weights, the hardest part of each weight becomes a 16-bit low-rank branch,
 * the residual is quantized to 4 bits; "Nunchaku Lite", quantization
 * walkthrough: the checkpoint is produced offline from the dense weights).
 * ------------------------------------------------------------------------- */

/*
 * svdq_calibrate_smooth -- the smoothing factor of one linear:
 *   lambda_k = bf16(sqrt(fl32(a_k / b_k))), a_k = max_m |x_cal[m, k]|,
 *   b_k = max_n |w[n, k]|; lambda_k = 1 when a_k or b_k is 0
 * (a migration of strength 1/2 between activations and weights).
 *   Mc, N, K    calibration rows, weight rows, channels; K even
 *   x_cal       bf16 [Mc, K] calibration activations
 *   w           bf16 [N, K] dense weight (nn.Linear layout)
 *   smooth_out  out bf16 [K]
 */
svdq_status svdq_calibrate_smooth(int64_t Mc, int64_t N, int64_t K, const void* x_cal, const void* w,
                                  void* smooth_out, void* stream);

/* Workspace bytes svdq_lowrank_decompose needs (-1 for unsupported sizes). */
int64_t svdq_lowrank_workspace_bytes(int64_t N, int64_t K, int rank, int oversample);

/*
 * svdq_lowrank_decompose -- the 16-bit low-rank branch and the residual:
 *   W_hat = w diag(smooth) (fp32, exact), so (X / lambda) W_hat^T = X w^T;
 *   the rank-`rank` approximation of W_hat by randomized subspace iteration
 *   (Halko, Martinsson and Tropp 2011, Algorithm 4.4): Y = W_hat Omega, then
 *   `iters` rounds of Z = orth(W_hat^T Q), Q = orth(W_hat Z) (CholeskyQR2), and
 *   Rayleigh-Ritz on B = Q^T W_hat (eigen-decomposition of B B^T) giving
 *   W_hat ~ U_r S_r V_r^T;
 *   l1t = bf16(L1^T), L1 = diag(1/lambda) V_r S_r^(1/2)   [rank, K] (applied to raw X)
 *   l2t = bf16(L2^T), L2 = S_r^(1/2) U_r^T                [N, rank]
 *   residual = W_hat - (diag(lambda) L1 L2)^T with the stored bf16 factors, fp32
 *   [N, K] (what svdq_quantize_weight turns into the 4-bit weight).
 *   rank        16, 32, 48 or 64; oversample >= 0 with rank + oversample <= 64
 *               and <= min(N, K); iters 0..64 (more = closer to the exact SVD)
 *   w           bf16 [N, K]; smooth bf16 [K] or NULL (lambda = 1); K % 64 == 0
 *   omega       fp32 [K, rank + oversample] test matrix (caller-drawn, e.g.
 *               standard normal)
 *   residual    out fp32 [N, K] (also the smoothed-weight workspace)
 *   work        device workspace of work_bytes >= svdq_lowrank_workspace_bytes()
 * The outputs depend on omega and on floating-point order; the product
 * L1 L2 approaches the exact rank-r truncation as iters grows.  A rank-deficient
 * W_hat is valid input: the first CholeskyQR pass shifts the Gram matrix's
 * diagonal by 1e-6 of its mean, so every pivot stays positive and the basis
 * vectors beyond the rank are rounding noise, to which Rayleigh-Ritz gives
 * singular values near zero (for a W_hat of rank below `rank`, L1 L2 reproduces
 * it).  A pivot that is not positive (an all-zero W_hat) zeroes its basis
 * vector, so an all-zero W_hat gives all-zero factors and residual.
 */
svdq_status svdq_lowrank_decompose(int64_t N, int64_t K, int rank, int oversample, int iters, const void* w,
                                   const void* smooth, const float* omega, void* l1t, void* l2t, float* residual,
                                   void* work, int64_t work_bytes, void* stream);

/*
 * svdq_lowrank_decompose_noalloc -- svdq_lowrank_decompose without the `work`
 * argument and without any allocation, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation).  Same arguments, kernels and results (bit for bit) as
 * svdq_lowrank_decompose; the workspace is the library's fixed per-GPU scratch
 * area of 16 MiB (held on each GPU the library runs on until the process
 * ends), so sizes whose svdq_lowrank_workspace_bytes() exceeds 16 MiB are
 * rejected with SVDQ_ERR_UNSUPPORTED.  Every call on a GPU uses that GPU's one
 * scratch area: calls that overlap on one GPU (on different streams, or from
 * several threads) race and must not be issued; calls in sequence on one
 * stream are fine (every part of the workspace is written before it is read).
 */
svdq_status svdq_lowrank_decompose_noalloc(int64_t N, int64_t K, int rank, int oversample, int iters,
                                           const void* w, const void* smooth, const float* omega, void* l1t,
                                           void* l2t, float* residual, void* stream);

/*
 * svdq_quantize_weight -- the 4-bit residual weight, per (row n, group):
 *   int4 (group 64):  s = fp16_sat(fl32(amax / 7)), q = clamp(rne(fl32(r * fl32(1/s))), -8, 7)
 *   nvfp4 (group 16): s = e4m3_sat(fl32(amax / fl32(6 * alpha_w))),
 *                     c = e2m1_sat(fl32(r * fl32(1 / fl32(s * alpha_w))))
 * (the activation quantizer's steps on an fp32 input, no smoothing).
 *   residual    fp32 [N, K], K % 64 == 0
 *   codes       out u8 [N, K/2]; scales out int4: fp16 [N, K/64], nvfp4: E4M3 u8 [N, K/16]
 */
svdq_status svdq_quantize_weight(int precision, int group_size, int64_t N, int64_t K, const float* residual,
                                 float w_global_scale, void* codes, void* scales, void* stream);

/*
 * awq_quantize_weight -- AWQ int4 weight-only quantization per (row, 64-group),
 * min-max over a range containing 0: lo = min(0, min w), hi = max(0, max w),
 * s = fp16(fl32((hi - lo) / 15)), z = clamp(rne(fl32(-lo * fl32(1/s))), 0, 15)
 * (fp16), q = clamp(rne(fl32(w * fl32(1/s))) + z, 0, 15); all-zero group:
 * s = z = 0, codes 0.  Output layout as awq_w4a16_gemv consumes it.
 *   w           bf16 [N, K], K % 64 == 0
 *   codes out u8 [N, K/2]; scales, zeros out fp16 [N, K/64]
 */
svdq_status awq_quantize_weight(int group_size, int64_t N, int64_t K, const void* w, void* codes, void* scales,
                                void* zeros, void* stream);

/*
 * svdq_w4a4_group_psums -- test support: the per-group partial products of
 * the 4-bit GEMM, P[m,n,g] = sum_{k in g} a_code * w_code, computed by the
 * same unpack and matrix-core path as svdq_w4a4_gemm.  int4: int32 (exact);
 * nvfp4: fp32 (exact: multiples of 1/4, |P| <= 576).  Layout [M, N, K/G],
 * g fastest.  Crops of larger operands are taken by pointer offsets (rows of
 * the code buffers are contiguous).  Shape limits as for svdq_w4a4_gemm.
 */
svdq_status svdq_w4a4_group_psums(int precision, int group_size, int64_t M, int64_t N,
                                  int64_t K, const void* act_codes, const void* w_codes,
                                  void* psums, void* stream);

/* Message for the last non-OK status returned on this thread ("" if none). */
const char* svdq_last_error(void);

/* ABI version of this header (bumped on any incompatible change). */
int svdq_abi_version(void);

/*
 * Test hook: when `arch` is non-NULL every later architecture check sees this
 * gcnArchName instead of the device's; NULL restores the real check.  Lets a
 * test prove that a non-gfx950 device gets SVDQ_ERR_UNSUPPORTED and no launch.
 */
void svdq_test_set_arch_override(const char* arch);

/*
 * Test hook: `on` != 0 makes every later int4 svdq_w4a4_gemm run its one-copy
 * kernel instance, also on a grid of at most one 128x128 tile per compute unit
 * (which otherwise runs a K-split instance: two copies of the workgroup, each
 * over half of K).  Lets a test compare both instances on a small shape; 0
 * restores the automatic choice.  Results differ between the instances only in
 * the fp32 summation order.
 */
void svdq_test_set_no_ksplit(int on);

#ifdef __cplusplus
}
#endif

#endif /* SVDQ_H_ */
