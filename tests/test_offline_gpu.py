"""Parity of the offline weight side on the GPU with the oracle, through the C ABI.

Bit-exact: the smoothing factor (column maxima, one division, one square
root), the residual quantizer on a given fp32 residual, the AWQ weight
quantizer.  The rank-r decomposition is a randomized iteration in fp32 against
the oracle's exact double SVD, so it is held to what is unique: the rank-r
product diag(lambda) L1 L2 (within 1e-2 relative Frobenius of the exact
truncation, the factors being bf16), the residual's norm (within 1% of the
optimum the exact truncation gives), and the decomposition's defining
identity X L1 L2 + (X / lambda) R^T = X W^T on the GPU's own outputs.
"""
import numpy as np
import pytest
import torch

import oracle
import bit_w4a4_quantized_smooth_amd as sq
from bit_w4a4_quantized_smooth_amd import synth

pytestmark = pytest.mark.gpu


def dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.view(dtype)
    return t.cuda()


def b16(bits):
    return dev(np.asarray(bits, np.uint16).view(np.int16), torch.bfloat16)


def bits(t):
    return t.cpu().view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("shape", [(512, 256, 256), (1000, 640, 384), (37, 130, 64)])
def test_calibrate_smooth_bit_exact(shape):
    N, K, Mc = shape
    print(f"[offline] calibrate {shape}", flush=True)
    d = synth.dense_layer(4001, N, K, Mc)
    lam = sq.calibrate_smooth(b16(d["x_cal"]), b16(d["w"]))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(lam), oracle.calibrate_smooth(d["x_cal"], d["w"]))


@pytest.mark.parametrize("prec", [sq.SVDQ_INT4, sq.SVDQ_NVFP4])
def test_quantize_weight_bit_exact(prec):
    print(f"[offline] quantize_weight prec {prec}", flush=True)
    rng = np.random.default_rng(4002)
    r = (rng.standard_normal((300, 512)) * rng.uniform(0.001, 0.05, (300, 1))).astype(np.float32)
    r[3, :64] = 0.0                       # an all-zero group
    r[5, 64:128] = 1e-6                   # tiny scales (fp16 / E4M3 subnormal range)
    alpha = 2.0 ** -7 if prec == sq.SVDQ_NVFP4 else 1.0
    codes, scales = sq.quantize_weight(prec, dev(r), alpha)
    torch.cuda.synchronize()
    oc, os_ = oracle.quantize_weight(prec, r, alpha)
    np.testing.assert_array_equal(codes.cpu().numpy(), oc)
    got_s = scales.cpu().view(torch.int16).numpy().view(np.uint16) if prec == sq.SVDQ_INT4 else scales.cpu().numpy()
    np.testing.assert_array_equal(got_s, os_)


def test_awq_quantize_weight_bit_exact():
    print("[offline] awq_quantize_weight", flush=True)
    d = synth.dense_layer(4003, 384, 1024)
    w = d["w"].copy()
    w[7, :64] = 0
    codes, scales, zeros = sq.awq_quantize_weight(b16(w))
    torch.cuda.synchronize()
    oc, os_, oz = oracle.awq_quantize_weight(w)
    np.testing.assert_array_equal(codes.cpu().numpy(), oc)
    np.testing.assert_array_equal(bits(scales), os_)
    np.testing.assert_array_equal(bits(zeros), oz)


@pytest.mark.parametrize("shape", [(1536, 768, 32), (640, 384, 16)])
def test_lowrank_decompose(shape):
    N, K, rank = shape
    print(f"[offline] lowrank {shape}", flush=True)
    d = synth.dense_layer(4004, N, K, planted_rank=rank)
    lam_b = oracle.calibrate_smooth(d["x_cal"], d["w"])
    omega = d["omega"][:, :rank + 16]
    l1t, l2t, res = sq.lowrank_decompose(b16(d["w"]), b16(lam_b), dev(omega), rank, iters=4)
    torch.cuda.synchronize()
    ref = oracle.lowrank_decompose(d["w"], lam_b, rank)
    lam = synth.bf16_bits_to_f64(lam_b)
    l1 = synth.bf16_bits_to_f64(bits(l1t)).T        # [K, r]
    l2 = synth.bf16_bits_to_f64(bits(l2t)).T        # [r, N]
    R = res.cpu().numpy().astype(np.float64)
    prod = ((lam[:, None] * l1) @ l2).T              # the branch in smoothed-weight space [N, K]
    e = np.linalg.norm(prod - ref["lowrank"]) / np.linalg.norm(ref["lowrank"])
    opt = np.linalg.norm(ref["residual"])
    print(f"[offline] rank-r product rel err {e:.3g}, residual {np.linalg.norm(R):.5g} vs {opt:.5g}", flush=True)
    assert e <= 1e-2
    assert np.linalg.norm(R) <= 1.01 * opt
    # the defining identity on the GPU's own outputs
    x = synth.bf16_bits_to_f64(d["x_cal"][:64])
    w = synth.bf16_bits_to_f64(d["w"])
    y = x @ l1 @ l2 + (x / lam[None, :]) @ R.T
    yref = x @ w.T
    assert np.max(np.abs(y - yref)) <= 1e-4 * np.max(np.abs(yref))


def test_offline_to_online_roundtrip():
    # calibrate -> decompose -> quantize the residual -> run the quantized layer:
    # the W4A4 output approximates the dense X W^T (4-bit weights and activations)
    print("[offline] roundtrip", flush=True)
    N, K, rank = 768, 512, 32
    d = synth.dense_layer(4005, N, K, planted_rank=rank)
    x = d["x_cal"][:128]
    lam = sq.calibrate_smooth(b16(d["x_cal"]), b16(d["w"]))
    l1t, l2t, res = sq.lowrank_decompose(b16(d["w"]), lam, dev(d["omega"]), rank, iters=4)
    wc, ws = sq.quantize_weight(sq.SVDQ_INT4, res)
    y = sq.svdq_linear(sq.SVDQ_INT4, b16(x), lam, l1t, wc, ws, l2t, None)
    torch.cuda.synchronize()
    yd = synth.bf16_bits_to_f64(x) @ synth.bf16_bits_to_f64(d["w"]).T
    e = np.linalg.norm(synth.bf16_bits_to_f64(bits(y)) - yd) / np.linalg.norm(yd)
    print(f"[offline] W4A4 layer vs dense: relative Frobenius error {e:.3g}", flush=True)
    assert e <= 0.1


@pytest.mark.parametrize("kind", ["rank8", "zero"])
def test_lowrank_decompose_rank_deficient(kind):
    # a weight of rank 8 decomposed at rank 16 (the branch reproduces it, the
    # residual is rounding), and an all-zero weight (zero factors, no NaN)
    N, K, rank = 640, 384, 16
    print(f"[offline] lowrank rank-deficient {kind}", flush=True)
    d = synth.dense_layer(4006, N, K, planted_rank=0)
    if kind == "rank8":
        g = np.random.default_rng(4007)
        w = (g.standard_normal((N, 8)) @ g.standard_normal((8, K))) * 0.05
    else:
        w = np.zeros((N, K))
    wb = synth.to_bf16_bits(w)
    lam_b = oracle.calibrate_smooth(d["x_cal"], wb)
    l1t, l2t, res = sq.lowrank_decompose(b16(wb), b16(lam_b), dev(d["omega"][:, :rank + 16]), rank, iters=4)
    torch.cuda.synchronize()
    l1 = synth.bf16_bits_to_f64(bits(l1t)).T
    l2 = synth.bf16_bits_to_f64(bits(l2t)).T
    R = res.cpu().numpy().astype(np.float64)
    lam = synth.bf16_bits_to_f64(lam_b)
    assert np.isfinite(l1).all() and np.isfinite(l2).all() and np.isfinite(R).all()
    w_hat = synth.bf16_bits_to_f64(wb) * lam[None, :]
    prod = ((lam[:, None] * l1) @ l2).T
    if kind == "zero":
        assert not prod.any() and not R.any()
    else:
        e = np.linalg.norm(prod - w_hat) / np.linalg.norm(w_hat)
        print(f"[offline] rank-8 weight: branch rel err {e:.3g}", flush=True)
        assert e <= 1e-2
        assert np.linalg.norm(R) <= 1e-2 * np.linalg.norm(w_hat)
