"""Pins of the oracle's method functions to things other than itself.

* hand-worked examples (tests/golden/worked_examples.json);
* invariants of absmax quantization: code range, the absmax channel hitting
  +-qmax, the half-step error bound, lossless round trip of grid-exact inputs,
  power-of-two scale equivariance, sign symmetry;
* library routines: numpy float32 division and float16 casts for the scale,
  numpy int64 sums for the group products, numpy float64 matmuls for the
  low-rank branch, the dequantized GEMM and the AWQ linear;
* special cases with closed forms: rank 0, all-zero weight codes, no bias,
  one-hot activations.

Each check is chosen so that a plausible slip in the oracle (qmax 8 instead
of 7, truncation instead of round-to-nearest-even, swapped nibbles, a dropped
scale, a transposed low-rank factor, a wrong zero-point sign) fails here.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
from bit_w4a4_quantized_smooth_amd import synth

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")))


# --- independent helpers (numpy only) -----------------------------------------
def unpack_signed(codes):
    lo = (codes & 0xF).astype(np.int64)
    hi = (codes >> 4).astype(np.int64)
    out = np.empty((codes.shape[0], codes.shape[1] * 2), np.int64)
    out[:, 0::2], out[:, 1::2] = lo, hi
    return np.where(out >= 8, out - 16, out)


def unpack_unsigned(codes):
    out = np.empty((codes.shape[0], codes.shape[1] * 2), np.int64)
    out[:, 0::2], out[:, 1::2] = codes & 0xF, codes >> 4
    return out


E2M1 = np.array([0, .5, 1, 1.5, 2, 3, 4, 6, -0.0, -.5, -1, -1.5, -2, -3, -4, -6])


def unpack_e2m1(codes):
    return E2M1[unpack_unsigned(codes)]


def bf16(a):
    return synth.to_bf16_bits(np.asarray(a, np.float64))


def bf16f(b):
    return synth.bf16_bits_to_f64(b)


def f16f(h):
    return np.asarray(h, np.uint16).view(np.float16).astype(np.float64)


def e4m3f(b):
    return torch.from_numpy(np.asarray(b, np.uint8)).view(torch.float8_e4m3fn).double().numpy()


def group_row(head, G):
    row = np.zeros(G)
    row[:len(head)] = head
    return row


# --- golden, hand-worked ---------------------------------------------------------
@pytest.mark.parametrize("name", ["int4_plain", "int4_smoothed", "int4_inexact_scale"])
def test_golden_int4_quantize(name):
    ex = GOLD[name]
    x = bf16(group_row(ex["x_head"], 64)[None, :])
    lam = None if ex["lambda_head"] is None else bf16(np.concatenate([ex["lambda_head"], np.ones(64 - len(ex["lambda_head"]))]))
    codes, scales = oracle.quantize_act(oracle.INT4, x, lam)
    assert int(scales[0, 0]) == ex["scale_bits"]
    head = ex["code_bytes_head"]
    assert list(codes[0, :len(head)]) == head
    assert not codes[0, len(head):].any()


def test_golden_nvfp4_quantize():
    ex = GOLD["nvfp4_plain"]
    x = bf16(group_row(ex["x_head"], 16)[None, :])
    codes, scales = oracle.quantize_act(oracle.NVFP4, x, None, alpha=ex["alpha"])
    assert int(scales[0, 0]) == ex["scale_bits"]
    head = ex["code_bytes_head"]
    assert list(codes[0, :len(head)]) == head and not codes[0, len(head):].any()


def _pack_signed(vals, K):
    q = np.zeros(K, np.int64)
    q[:len(vals)] = vals
    return synth.pack_nibbles((q & 0xF)[None, :])


def test_golden_int4_linear_and_psum():
    ex = GOLD["int4_linear"]
    a = _pack_signed(ex["a_codes_head"], 64)
    w = _pack_signed(ex["w_codes_head"], 64)
    sa = np.array([[np.float16(ex["a_scale"])]]).view(np.uint16)
    sw = np.array([[np.float16(ex["w_scale"])]]).view(np.uint16)
    assert oracle.group_psums(oracle.INT4, a, w)[0, 0, 0] == ex["psum"]
    r = ex["rank"]
    xl1 = np.zeros((1, r), np.float32)
    xl1[0, :len(ex["xl1_head"])] = ex["xl1_head"]
    l2t = bf16(group_row(ex["l2_head"], r)[None, :])
    bias = bf16([ex["bias"]])
    y, yb = oracle.w4a4_linear(oracle.INT4, a, sa, w, sw, xl1, l2t, bias)
    assert y[0, 0] == ex["y"] and yb[0, 0] == ex["y_bf16_bits"]
    y0, yb0 = oracle.w4a4_linear(oracle.INT4, a, sa, w, sw, None, None, bias)
    assert y0[0, 0] == ex["y_rank0"] and yb0[0, 0] == ex["y_rank0_bf16_bits"]


def test_golden_awq():
    ex = GOLD["awq_linear"]
    x = bf16(group_row(ex["x_head"], 64)[None, :])
    q = np.zeros((1, 64), np.int64)
    q[0, :3] = ex["codes_head"]
    codes = synth.pack_nibbles(q)
    s = np.array([[np.float16(ex["scale"])]]).view(np.uint16)
    z = np.array([[np.float16(ex["zero"])]]).view(np.uint16)
    y, _ = oracle.awq_linear(x, codes, s, z)
    assert y[0, 0] == ex["y"]


# --- int4 quantizer invariants -----------------------------------------------------
@pytest.fixture(scope="module")
def c1():
    return synth.svdq_layer(1001, 256, 512, 512, 16, synth.INT4, 0.01, 20.0)


def _smoothed_f32(x, lam):
    xf = bf16f(x).astype(np.float32)
    if lam is None:
        return xf
    r = (np.float32(1.0) / bf16f(lam).astype(np.float32)).astype(np.float32)
    return (xf * r[None, :]).astype(np.float32)


def test_int4_scale_matches_library_rounding(c1):
    codes, scales = oracle.quantize_act(oracle.INT4, c1["x"], c1["lam"])
    xh = _smoothed_f32(c1["x"], c1["lam"])
    amax = np.abs(xh).reshape(xh.shape[0], -1, 64).max(axis=2)
    with np.errstate(over="ignore"):
        ref = (amax / np.float32(7.0)).astype(np.float32).astype(np.float16)
    ref = np.where(np.isinf(ref), np.float16(65504), ref).view(np.uint16)
    assert np.array_equal(scales, ref)


def test_int4_code_range_and_absmax_hits_qmax(c1):
    codes, scales = oracle.quantize_act(oracle.INT4, c1["x"], c1["lam"])
    q = unpack_signed(codes)
    s = f16f(scales)
    assert q.min() >= -8 and q.max() <= 7
    normal = s >= 2.0 ** -14
    qg = q.reshape(q.shape[0], -1, 64)
    assert np.all(np.abs(qg[normal]) <= 7)
    xh = _smoothed_f32(c1["x"], c1["lam"]).reshape(qg.shape)
    idx = np.abs(xh).argmax(axis=2)
    at_max = np.take_along_axis(qg, idx[..., None], axis=2)[..., 0]
    assert np.all(np.abs(at_max[normal]) == 7)


def test_int4_half_step_error_bound(c1):
    codes, scales = oracle.quantize_act(oracle.INT4, c1["x"], c1["lam"])
    q = unpack_signed(codes).reshape(codes.shape[0], -1, 64)
    s = f16f(scales)[..., None]
    xh = _smoothed_f32(c1["x"], c1["lam"]).astype(np.float64).reshape(q.shape)
    err = np.abs(xh - q * s)
    assert np.all(err <= s * (0.5 + 2.0 ** -20))


def test_int4_grid_exact_roundtrip():
    rng = np.random.default_rng(5)
    M, K = 16, 256
    q = rng.integers(-7, 8, size=(M, K))
    q[:, ::64] = 7  # every group contains +7
    e = rng.integers(-6, 6, size=(M, K // 64))
    x = q * np.repeat(2.0 ** (-e.astype(np.float64)), 64, axis=1)
    codes, scales = oracle.quantize_act(oracle.INT4, bf16(x), None)
    assert np.array_equal(unpack_signed(codes), q)
    assert np.array_equal(f16f(scales), 2.0 ** (-e.astype(np.float64)))


def test_int4_scale_equivariance_and_sign_symmetry(c1):
    codes, scales = oracle.quantize_act(oracle.INT4, c1["x"], c1["lam"])
    lam2 = bf16(bf16f(c1["lam"]) * 4.0)
    codes2, scales2 = oracle.quantize_act(oracle.INT4, c1["x"], lam2)
    assert np.array_equal(codes, codes2)
    assert np.array_equal(f16f(scales2), f16f(scales) / 4.0)
    neg = (c1["x"] ^ np.uint16(0x8000)).astype(np.uint16)
    codes3, scales3 = oracle.quantize_act(oracle.INT4, neg, c1["lam"])
    assert np.array_equal(scales3, scales)
    assert np.array_equal(unpack_signed(codes3), -unpack_signed(codes))


def test_int4_zero_group_and_subnormal_scale_clamp():
    x = np.zeros((2, 128))
    x[1, :64] = 1e-6 * np.linspace(-1, 1, 64)  # fp16-subnormal scale
    x[1, 64:] = np.linspace(-3, 3, 64)
    codes, scales = oracle.quantize_act(oracle.INT4, bf16(x), None)
    q = unpack_signed(codes)
    assert not q[0].any() and not scales[0].any()
    assert q[1].min() >= -8 and q[1].max() <= 7
    s = f16f(scales[1, 0])
    assert 0 < s < 2.0 ** -14
    xh = bf16f(bf16(x))[1, :64]
    # against the stored (coarse) subnormal scale the codes still land within a step
    assert np.all(np.abs(xh - q[1, :64] * s) <= s * 0.5 + 1e-12) or q[1, :64].min() == -8


# --- nvfp4 quantizer invariants ------------------------------------------------------
@pytest.fixture(scope="module")
def c4small():
    return synth.svdq_layer(1004, 128, 256, 512, 32, synth.NVFP4, 0.005, 30.0)


def test_nvfp4_scale_matches_library_rounding(c4small):
    d = c4small
    codes, scales = oracle.quantize_act(oracle.NVFP4, d["x"], d["lam"], alpha=d["alpha_a"])
    xh = _smoothed_f32(d["x"], d["lam"])
    amax = np.abs(xh).reshape(xh.shape[0], -1, 16).max(axis=2)
    den = np.float32(np.float32(6.0) * np.float32(d["alpha_a"]))
    ref = torch.from_numpy((amax / den).astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(scales, ref)


def test_nvfp4_codes_on_grid_with_error_bound(c4small):
    d = c4small
    codes, scales = oracle.quantize_act(oracle.NVFP4, d["x"], d["lam"], alpha=d["alpha_a"])
    v = unpack_e2m1(codes).reshape(codes.shape[0], -1, 16)
    s = e4m3f(scales)[..., None] * np.float64(np.float32(d["alpha_a"]))
    xh = _smoothed_f32(d["x"], d["lam"]).astype(np.float64).reshape(v.shape)
    u = np.abs(xh) / np.where(s == 0, 1, s)
    # half the local E2M1 spacing (0.25 below 2, 0.5 below 4, 1 up to 6), plus
    # the rounding of the fp32 reciprocal and product
    half = np.where(u < 2, 0.25, np.where(u < 4, 0.5, 1.0))
    err = np.abs(u - np.abs(v))
    ok = (s == 0) | (err <= half * (1 + 2.0 ** -20) + 6 * 2.0 ** -22)
    assert np.all(ok)
    # the absmax element of every group with a nonzero scale maps to +-6 or +-4
    # (E4M3 rounding of the scale moves it at most 1/16 relative)
    idx = np.abs(xh).argmax(axis=2)
    at = np.take_along_axis(np.abs(v), idx[..., None], axis=2)[..., 0]
    assert np.all(at[s[..., 0] > 0] >= 4.0)


def test_nvfp4_sign_symmetry(c4small):
    d = c4small
    codes, scales = oracle.quantize_act(oracle.NVFP4, d["x"], d["lam"], alpha=d["alpha_a"])
    neg = (d["x"] ^ np.uint16(0x8000)).astype(np.uint16)
    codes2, scales2 = oracle.quantize_act(oracle.NVFP4, neg, d["lam"], alpha=d["alpha_a"])
    assert np.array_equal(scales, scales2)
    assert np.array_equal(unpack_e2m1(codes2), -unpack_e2m1(codes))


# --- products, low rank, the linear ---------------------------------------------
def test_int4_psums_against_numpy(c1):
    codes, _ = oracle.quantize_act(oracle.INT4, c1["x"], c1["lam"])
    P = oracle.group_psums(oracle.INT4, codes[:64], c1["w_codes"][:96])
    qa = unpack_signed(codes[:64]).reshape(64, -1, 64)
    qw = unpack_signed(c1["w_codes"][:96]).reshape(96, -1, 64)
    ref = np.einsum("mgk,ngk->mng", qa, qw)
    assert np.array_equal(P, ref)


def test_nvfp4_psums_against_numpy(c4small):
    d = c4small
    codes, _ = oracle.quantize_act(oracle.NVFP4, d["x"], d["lam"], alpha=d["alpha_a"])
    P = oracle.group_psums(oracle.NVFP4, codes[:32], d["w_codes"][:48])
    va = unpack_e2m1(codes[:32]).reshape(32, -1, 16)
    vw = unpack_e2m1(d["w_codes"][:48]).reshape(48, -1, 16)
    ref = np.einsum("mgk,ngk->mng", va, vw)
    assert np.array_equal(P.astype(np.float64), ref)


def test_lowrank_down_against_numpy(c1):
    xl1 = oracle.lowrank_down(c1["x"], c1["l1t"])
    ref = bf16f(c1["x"]) @ bf16f(c1["l1t"]).T
    assert np.allclose(xl1, ref, rtol=1e-6, atol=1e-6 * np.abs(ref).max())


def _dequant_y(a_vals, a_s, w_vals, w_s, G, xl1, l2t, bias, alpha=1.0):
    A = a_vals * np.repeat(a_s, G, axis=1)
    W = w_vals * np.repeat(w_s, G, axis=1)
    y = alpha * (A @ W.T)
    if xl1 is not None:
        y = y + xl1.astype(np.float64) @ bf16f(l2t).T
    if bias is not None:
        y = y + bf16f(bias)[None, :]
    return y


def test_int4_linear_equals_dequantized_matmul(c1):
    codes, scales = oracle.quantize_act(oracle.INT4, c1["x"], c1["lam"])
    xl1 = oracle.lowrank_down(c1["x"], c1["l1t"])
    y, yb = oracle.w4a4_linear(oracle.INT4, codes, scales, c1["w_codes"], c1["w_scales"], xl1,
                               c1["l2t"], c1["bias"])
    ref = _dequant_y(unpack_signed(codes), f16f(scales), unpack_signed(c1["w_codes"]),
                     f16f(c1["w_scales"]), 64, xl1, c1["l2t"], c1["bias"])
    assert np.max(np.abs(y - ref)) <= 1e-12 * np.max(np.abs(ref))
    assert np.array_equal(yb, bf16(y))
    # sampled evaluation equals the full grid
    rows = np.array([0, 5, 255, 100]); cols = np.array([511, 0, 7, 300])
    ys, _ = oracle.w4a4_linear(oracle.INT4, codes, scales, c1["w_codes"], c1["w_scales"], xl1,
                               c1["l2t"], c1["bias"], rows=rows, cols=cols)
    assert np.array_equal(ys, y[rows, cols])


def test_nvfp4_linear_equals_dequantized_matmul(c4small):
    d = c4small
    codes, scales = oracle.quantize_act(oracle.NVFP4, d["x"], d["lam"], alpha=d["alpha_a"])
    xl1 = oracle.lowrank_down(d["x"], d["l1t"])
    y, _ = oracle.w4a4_linear(oracle.NVFP4, codes, scales, d["w_codes"], d["w_scales"], xl1,
                              d["l2t"], d["bias"], alpha_a=d["alpha_a"], alpha_w=d["alpha_w"])
    ref = _dequant_y(unpack_e2m1(codes), e4m3f(scales), unpack_e2m1(d["w_codes"]),
                     e4m3f(d["w_scales"]), 16, xl1, d["l2t"], d["bias"],
                     alpha=np.float64(np.float32(d["alpha_a"])) * np.float64(np.float32(d["alpha_w"])))
    assert np.max(np.abs(y - ref)) <= 1e-12 * np.max(np.abs(ref))


def test_int4_linear_special_cases(c1):
    codes, scales = oracle.quantize_act(oracle.INT4, c1["x"], c1["lam"])
    xl1 = oracle.lowrank_down(c1["x"], c1["l1t"])
    # rank 0 == plain quantized GEMM (dequantized matmul, no low-rank term)
    y0, _ = oracle.w4a4_linear(oracle.INT4, codes, scales, c1["w_codes"], c1["w_scales"], None, None, None)
    ref0 = _dequant_y(unpack_signed(codes), f16f(scales), unpack_signed(c1["w_codes"]),
                      f16f(c1["w_scales"]), 64, None, None, None)
    assert np.max(np.abs(y0 - ref0)) <= 1e-12 * np.max(np.abs(ref0))
    # all-zero weight codes: y = XL1 . L2 + bias exactly as a numpy matmul
    zw = np.zeros_like(c1["w_codes"])
    yz, _ = oracle.w4a4_linear(oracle.INT4, codes, scales, zw, c1["w_scales"], xl1, c1["l2t"], c1["bias"])
    refz = xl1.astype(np.float64) @ bf16f(c1["l2t"]).T + bf16f(c1["bias"])[None, :]
    assert np.max(np.abs(yz - refz)) <= 1e-12 * np.max(np.abs(refz))
    # bias NULL equals bias 0
    yn, _ = oracle.w4a4_linear(oracle.INT4, codes, scales, c1["w_codes"], c1["w_scales"], xl1, c1["l2t"], None)
    yb0, _ = oracle.w4a4_linear(oracle.INT4, codes, scales, c1["w_codes"], c1["w_scales"], xl1, c1["l2t"],
                                np.zeros(512, np.uint16))
    assert np.array_equal(yn, yb0)


# --- AWQ ------------------------------------------------------------------------------
@pytest.fixture(scope="module")
def awq_small():
    return synth.awq_layer(1005, 4, 192, 512)


def test_awq_against_numpy(awq_small):
    d = awq_small
    y, yb = oracle.awq_linear(d["x"], d["w_codes"], d["w_scales"], d["w_zeros"], d["bias"])
    q = unpack_unsigned(d["w_codes"]).astype(np.float64)
    W = (q - np.repeat(f16f(d["w_zeros"]), 64, axis=1)) * np.repeat(f16f(d["w_scales"]), 64, axis=1)
    ref = bf16f(d["x"]) @ W.T + bf16f(d["bias"])[None, :]
    assert np.max(np.abs(y - ref)) <= 1e-12 * np.max(np.abs(ref))
    assert np.array_equal(yb, bf16(y))


def test_awq_special_cases(awq_small):
    d = awq_small
    N, K = d["N"], d["K"]
    # z = 8, s = 1: the weight is the signed code q - 8
    s1 = np.full((N, K // 64), np.float16(1.0)).view(np.uint16)
    z8 = np.full((N, K // 64), np.float16(8.0)).view(np.uint16)
    y, _ = oracle.awq_linear(d["x"], d["w_codes"], s1, z8)
    ref = bf16f(d["x"]) @ (unpack_unsigned(d["w_codes"]) - 8.0).T
    assert np.max(np.abs(y - ref)) <= 1e-12 * np.max(np.abs(ref))
    # one-hot x picks one dequantized weight column
    k = 77
    x1 = np.zeros((1, K)); x1[0, k] = 1.0
    y1, _ = oracle.awq_linear(bf16(x1), d["w_codes"], d["w_scales"], d["w_zeros"])
    col = (unpack_unsigned(d["w_codes"])[:, k] - f16f(d["w_zeros"])[:, k // 64]) * f16f(d["w_scales"])[:, k // 64]
    assert np.array_equal(y1[0], col)
