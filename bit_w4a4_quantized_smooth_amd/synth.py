"""Seeded synthetic inputs for the SVDQuant W4A4 linear and the AWQ W4A16 linear.

This module only makes inputs: random draws, storage-format conversion through
library casts (numpy / torch CPU), nibble packing of the given weight codes and
the offline calibration statistics (the smoothing factor lambda and the NVFP4
per-tensor activation scale).  It holds none of the method's quantize, product
or dequantize arithmetic; both the HIP path and the CPU oracle consume the
same bytes from it.

Shapes follow the workloads of the pages: diffusion-transformer projections at
hidden size 3072 with 4096 image + 512 text tokens for a 1024x1024 image (the
pages' examples run 1024x1024 generation; "Nunchaku Lite", loading example),
the fused Q/K/V projection (Q, K, V concatenated along the output dimension;
blog "Nunchaku 4-bit inference in Diffusers", structural rewrites section),
the GELU MLP pair, and the memory-bound modulation projection served by
awq_w4a16 ("Introducing Nunchaku Lite").  No trained weights or calibration
data exist here, so every tensor is drawn from the distribution stated below.

Conventions: bf16 / fp16 arrays are uint16 bit patterns, E4M3 arrays uint8,
4-bit codes are packed two per byte with the even channel in the low nibble.
Low-rank factors are stored in nn.Linear layout: l1t = L1^T [r, K] and
l2t = L2^T [N, r].
"""
from __future__ import annotations

import numpy as np
import torch

INT4, NVFP4 = 0, 1


def _rng(seed: int, tensor_id: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tensor_id])))


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(b, dtype=np.uint16).view(np.int16)).view(torch.bfloat16)
    return t.to(torch.float64).numpy()


def to_f16_bits(a: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float64).astype(np.float16).view(np.uint16)


def to_e4m3_bits(a: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy().copy()


def pack_nibbles(n: np.ndarray) -> np.ndarray:
    """[rows, K] array of 4-bit values (0..15) -> packed uint8 [rows, K/2]."""
    n = np.asarray(n, dtype=np.uint8) & 0xF
    return np.ascontiguousarray(n[:, 0::2] | (n[:, 1::2] << 4))


def activations(seed: int, M: int, K: int, outlier_frac: float, outlier_scale: float,
                kind: str = "normal", tensor_id: int = 1) -> np.ndarray:
    """bf16 bits [M, K]: N(0,1) (or GELU_erf of N(0,1)) with a seeded set of
    round(outlier_frac*K) channels multiplied by outlier_scale."""
    g = _rng(seed, tensor_id)
    x = g.standard_normal((M, K))
    if kind == "gelu":
        x = torch.nn.functional.gelu(torch.from_numpy(x), approximate="none").numpy()
    n_out = int(round(outlier_frac * K))
    if n_out:
        ch = _rng(seed, tensor_id + 100).choice(K, size=n_out, replace=False)
        x[:, ch] *= outlier_scale
    return to_bf16_bits(x)


def smoothing_factor(x_bits: np.ndarray) -> np.ndarray:
    """Per-channel smoothing factor lambda_k = bf16(sqrt(max_m |X_mk|)), 1 where
    the column is all zero (offline calibration statistic)."""
    xa = np.abs(bf16_bits_to_f64(x_bits)).max(axis=0) if x_bits.shape[0] else np.zeros(x_bits.shape[1])
    lam = np.sqrt(xa)
    lam[lam == 0] = 1.0
    return to_bf16_bits(lam)


def nvfp4_act_global_scale(x_bits: np.ndarray, lam_bits: np.ndarray | None) -> float:
    """Static per-tensor NVFP4 activation scale: max |X/lambda| / (6*448),
    computed in double from the calibration batch and stored as fp32."""
    xf = np.abs(bf16_bits_to_f64(x_bits))
    if lam_bits is not None:
        xf = xf / bf16_bits_to_f64(lam_bits)[None, :]
    amax = float(xf.max()) if xf.size else 0.0
    return float(np.float32(amax / (6.0 * 448.0))) if amax > 0 else 1.0


def svdq_layer(seed: int, M: int, N: int, K: int, rank: int, prec: int = INT4,
               outlier_frac: float = 0.01, outlier_scale: float = 20.0, kind: str = "normal",
               smooth: bool = True, with_bias: bool = True, alpha_w: float = 2.0 ** -6) -> dict:
    """All inputs of one svdq_w4a4 linear.

    int4:  W codes uniform integers in [-8, 7] (two's complement nibbles),
           W scales fp16 ~ U(0.005, 0.02) per (row, 64-group).
    nvfp4: W codes uniform over the 16 E2M1 nibbles, W scales
           e4m3(U(0.005, 0.02) / alpha_w) per (row, 16-group), alpha_w = 2^-6.
    L1 [K, r], L2 [r, N] bf16 ~ N(0, 0.02^2); bias bf16 ~ N(0, 0.01^2).
    """
    G = 64 if prec == INT4 else 16
    x = activations(seed, M, K, outlier_frac, outlier_scale, kind)
    lam = smoothing_factor(x) if smooth else None
    gw = _rng(seed, 3)
    if prec == INT4:
        wq = gw.integers(-8, 8, size=(N, K))
        w_codes = pack_nibbles(wq & 0xF)
        w_scales = to_f16_bits(_rng(seed, 4).uniform(0.005, 0.02, size=(N, K // G)))
        alpha_a = 1.0
        alpha_w_out = 1.0
    else:
        w_codes = pack_nibbles(gw.integers(0, 16, size=(N, K)))
        w_scales = to_e4m3_bits(_rng(seed, 4).uniform(0.005, 0.02, size=(N, K // G)) / alpha_w)
        alpha_a = nvfp4_act_global_scale(x, lam)
        alpha_w_out = float(np.float32(alpha_w))
    l1t = to_bf16_bits(_rng(seed, 5).normal(0.0, 0.02, size=(K, rank)).T) if rank else np.zeros((0, K), np.uint16)
    l2t = to_bf16_bits(_rng(seed, 6).normal(0.0, 0.02, size=(rank, N)).T) if rank else np.zeros((N, 0), np.uint16)
    bias = to_bf16_bits(_rng(seed, 7).normal(0.0, 0.01, size=N)) if with_bias else None
    return dict(prec=prec, group=G, M=M, N=N, K=K, rank=rank, x=x, lam=lam,
                w_codes=w_codes, w_scales=w_scales, alpha_a=alpha_a, alpha_w=alpha_w_out,
                l1t=np.ascontiguousarray(l1t), l2t=np.ascontiguousarray(l2t), bias=bias)


def rope_table(S: int, head_dim: int, base: float = 10000.0) -> np.ndarray:
    """fp32 [S, head_dim/2, 2] (cos, sin) pairs of the angles s * base^(-2p/head_dim) for
    token positions s = 0..S-1 and channel pairs p: a standard rotary table (the
    operator takes any table of (cos, sin) pairs as an input)."""
    s = np.arange(S, dtype=np.float64)[:, None]
    p = np.arange(head_dim // 2, dtype=np.float64)[None, :]
    ang = s * base ** (-2.0 * p / head_dim)
    return np.ascontiguousarray(np.stack([np.cos(ang), np.sin(ang)], axis=-1).astype(np.float32))


def qkv_layer(seed: int, M: int, heads: int, head_dim: int, K: int, rank: int, prec: int = INT4,
              outlier_frac: float = 0.01, outlier_scale: float = 20.0, S: int | None = None,
              with_rope: bool = True, with_bias: bool = True) -> dict:
    """All inputs of the fused attention projection: an svdq_w4a4 linear with
    N = 3 * heads * head_dim (Q, K, V weights concatenated in that order), per-head
    RMSNorm weights norm_q, norm_k bf16 ~ U(0.5, 1.5) [head_dim], eps = 1e-6, and a
    rotary table for S positions (default S = M: one sequence)."""
    d = svdq_layer(seed, M, 3 * heads * head_dim, K, rank, prec, outlier_frac, outlier_scale,
                   with_bias=with_bias)
    d.update(heads=heads, head_dim=head_dim,
             norm_q=to_bf16_bits(_rng(seed, 9).uniform(0.5, 1.5, head_dim)),
             norm_k=to_bf16_bits(_rng(seed, 10).uniform(0.5, 1.5, head_dim)),
             eps=1e-6, rope=rope_table(S if S is not None else M, head_dim) if with_rope else None)
    return d


def mlp_layer(seed: int, M: int, hidden: int, dim: int, rank: int, prec: int = INT4) -> dict:
    """The two linears of a DiT MLP (dim -> hidden -> dim) for the fused up-projection:
    `up` = svdq_layer(seed, M, hidden, dim, rank, prec) (its X, outliers and weights); the
    down projection's smoothing factor lam_down bf16 ~ U(0.5, 2) [hidden] (a stand-in for a
    calibrated one: calibration would need the hidden activations, which only the method
    computes), its L1^T bf16 ~ N(0, 0.02^2) [rank, hidden] and its weights as in
    svdq_layer (int4: codes uniform in [-8, 7], fp16 scales ~ U(0.005, 0.02); nvfp4: codes
    uniform over the 16 E2M1 nibbles, scales e4m3(U(0.005, 0.02) / alpha_w), alpha_w = 2^-6),
    L2^T and bias.  nvfp4: the down projection's activation global scale alpha_a = 2^-6, a
    stand-in for a calibrated one for the same reason as lam_down (it keeps amax / (6 alpha)
    of these hidden activations inside the E4M3 range)."""
    up = svdq_layer(seed, M, hidden, dim, rank, prec, 0.005, 30.0)
    g = 64 if prec == INT4 else 16
    if prec == INT4:
        w_codes = pack_nibbles(_rng(seed, 23).integers(-8, 8, size=(dim, hidden)) & 0xF)
        w_scales = to_f16_bits(_rng(seed, 24).uniform(0.005, 0.02, size=(dim, hidden // g)))
        alpha_a, alpha_w = 1.0, 1.0
    else:
        aw = 2.0 ** -6
        w_codes = pack_nibbles(_rng(seed, 23).integers(0, 16, size=(dim, hidden)))
        w_scales = to_e4m3_bits(_rng(seed, 24).uniform(0.005, 0.02, size=(dim, hidden // g)) / aw)
        alpha_a, alpha_w = 2.0 ** -6, aw
    down = dict(
        prec=prec,
        lam=to_bf16_bits(_rng(seed, 21).uniform(0.5, 2.0, hidden)),
        l1t=to_bf16_bits(_rng(seed, 22).normal(0.0, 0.02, size=(rank, hidden))) if rank else np.zeros((0, hidden), np.uint16),
        w_codes=w_codes, w_scales=w_scales, alpha_a=alpha_a, alpha_w=alpha_w,
        l2t=to_bf16_bits(_rng(seed, 25).normal(0.0, 0.02, size=(dim, rank))) if rank else np.zeros((dim, 0), np.uint16),
        bias=to_bf16_bits(_rng(seed, 26).normal(0.0, 0.01, size=dim)),
        rank=rank, N=dim, K=hidden)
    return dict(up=up, down=down)


def dense_layer(seed: int, N: int, K: int, Mc: int = 256, planted_rank: int = 32) -> dict:
    """A dense bf16 weight and a calibration batch for the offline weight side:
    w = N(0, 0.02^2) noise + a planted rank-`planted_rank` part whose singular values
    e * (3 + 5 exp(-i/16)) stand well above the noise's largest singular value
    e = 0.02 (sqrt N + sqrt K) (random orthonormal directions): a weight whose hardest
    part a low-rank branch can carry; x_cal bf16 [Mc, K] ~ N(0, 1) with 1% of the
    channels multiplied by 25 (activation outliers); omega fp32 [K, 48] ~ N(0, 1), the
    test matrix of the randomized range finder (48 = rank 32 + oversampling 16)."""
    g = _rng(seed, 31)
    w = g.standard_normal((N, K)) * 0.02
    if planted_rank:
        u, _ = np.linalg.qr(_rng(seed, 32).standard_normal((N, planted_rank)))
        v, _ = np.linalg.qr(_rng(seed, 33).standard_normal((K, planted_rank)))
        e = 0.02 * (np.sqrt(N) + np.sqrt(K))
        s = e * (3.0 + 5.0 * np.exp(-np.arange(planted_rank) / 16.0))
        w += (u * s[None, :]) @ v.T
    x = _rng(seed, 34).standard_normal((Mc, K))
    ch = _rng(seed, 35).choice(K, size=max(1, K // 100), replace=False)
    x[:, ch] *= 25.0
    omega = _rng(seed, 36).standard_normal((K, 48)).astype(np.float32)
    return dict(w=to_bf16_bits(w), x_cal=to_bf16_bits(x), omega=omega, N=N, K=K)


def awq_layer(seed: int, M: int, N: int, K: int, with_bias: bool = True) -> dict:
    """All inputs of one awq_w4a16 linear: x bf16 ~ N(0,1) [M, K]; unsigned codes
    uniform in 0..15 [N, K]; fp16 scales ~ U(0.005, 0.02) and fp16 zero-points
    that are uniform integers in 0..15, per (row, 64-group); bias ~ N(0, 0.01^2)."""
    G = 64
    x = to_bf16_bits(_rng(seed, 1).standard_normal((M, K)))
    w_codes = pack_nibbles(_rng(seed, 3).integers(0, 16, size=(N, K)))
    w_scales = to_f16_bits(_rng(seed, 4).uniform(0.005, 0.02, size=(N, K // G)))
    w_zeros = to_f16_bits(_rng(seed, 8).integers(0, 16, size=(N, K // G)).astype(np.float64))
    bias = to_bf16_bits(_rng(seed, 7).normal(0.0, 0.01, size=N)) if with_bias else None
    return dict(M=M, N=N, K=K, group=G, x=x, w_codes=w_codes, w_scales=w_scales,
                w_zeros=w_zeros, bias=bias)


# The five workloads (seeds 1001..1005).  Each entry builds its inputs on call.
WORKLOADS = {
    "svdq_int4_256x512x512_r16": lambda: svdq_layer(1001, 256, 512, 512, 16, INT4, 0.01, 20.0),
    "dit_qkv_int4_4608x9216x3072_r32": lambda: svdq_layer(1002, 4608, 9216, 3072, 32, INT4, 0.005, 30.0),
    "dit_mlp_up_int4_4608x12288x3072_r32": lambda: svdq_layer(1002, 4608, 12288, 3072, 32, INT4, 0.005, 30.0),
    "dit_mlp_down_int4_4608x3072x12288_r32": lambda: svdq_layer(1003, 4608, 3072, 12288, 32, INT4, 0.0, 1.0, "gelu"),
    "dit_qkv_nvfp4_4608x9216x3072_r32": lambda: svdq_layer(1004, 4608, 9216, 3072, 32, NVFP4, 0.005, 30.0),
    "awq_mod_2x18432x3072": lambda: awq_layer(1005, 2, 18432, 3072),
    "awq_mod_64x18432x3072": lambda: awq_layer(1005, 64, 18432, 3072),
}
