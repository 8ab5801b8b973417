"""Pins of the oracle's offline weight side: smoothing-factor calibration,
the rank-r decomposition of the smoothed weight, residual quantization and
AWQ weight quantization, against hand-worked cases, exact identities (the
decomposition must reproduce X W^T exactly in double, which fixes the
direction of the smoothing and where 1/lambda goes) and cross-checks with the
independently written activation quantizer."""
import numpy as np
import pytest

import oracle
from bit_w4a4_quantized_smooth_amd import synth


def bf(a):
    return synth.to_bf16_bits(np.asarray(a, np.float64))


def f(bits):
    return synth.bf16_bits_to_f64(bits)


def test_calibrate_smooth_hand_cases():
    K = 5
    x = np.zeros((3, K))
    w = np.zeros((4, K))
    x[1, 0], w[2, 0] = -4.0, 1.0    # sqrt(4 / 1) = 2
    x[0, 1], w[0, 1] = 0.5, -8.0    # sqrt(1/16) = 0.25
    x[2, 2], w[3, 2] = 2.0, 1.0     # sqrt(2) -> bf16 1.4140625
    w[1, 3] = 3.0                   # no activation: 1
    x[0, 4] = 7.0                   # no weight: 1
    lam = oracle.calibrate_smooth(bf(x), bf(w))
    np.testing.assert_array_equal(f(lam), [2.0, 0.25, 1.4140625, 1.0, 1.0])


def _weights(seed, N, K, rank_planted=None):
    rng = np.random.default_rng(seed)
    w = rng.standard_normal((N, K)) * 0.02
    if rank_planted:
        w += rng.standard_normal((N, rank_planted)) @ rng.standard_normal((rank_planted, K)) * 0.05
    x = rng.standard_normal((32, K))
    x[:, rng.choice(K, 4, replace=False)] *= 25.0  # outlier channels
    return bf(w), bf(x)


def test_decomposition_reproduces_the_layer_exactly():
    w, x = _weights(1, 96, 128, 8)
    lam = oracle.calibrate_smooth(x, w)
    d = oracle.lowrank_decompose(w, lam, 16)
    xf, wf, lamf = f(x), f(w), f(lam)
    l1 = f(d["l1t"]).T
    l2 = f(d["l2t"]).T
    # low-rank branch on raw X plus the residual on X / lambda == X W^T
    y = xf @ l1 @ l2 + (xf / lamf[None, :]) @ d["residual"].T
    np.testing.assert_allclose(y, xf @ wf.T, rtol=0, atol=1e-10 * np.abs(xf @ wf.T).max())
    # the branch really carries the top of the smoothed weight: residual << smoothed weight
    assert np.linalg.norm(d["residual"]) < 0.5 * np.linalg.norm(d["w_hat"])


def test_lowrank_is_the_best_rank_r_approximation():
    w, x = _weights(2, 80, 64)
    lam = oracle.calibrate_smooth(x, w)
    d = oracle.lowrank_decompose(w, lam, 8)
    err = np.linalg.norm(d["w_hat"] - d["lowrank"])
    # Eckart-Young: the error is the energy of the dropped singular values
    np.testing.assert_allclose(err ** 2, np.sum(d["sigma"][8:] ** 2), rtol=1e-9)
    # and no random rank-8 projection does better
    rng = np.random.default_rng(3)
    for _ in range(5):
        q, _ = np.linalg.qr(rng.standard_normal((80, 8)))
        assert np.linalg.norm(d["w_hat"] - q @ (q.T @ d["w_hat"])) > err
    # an exactly rank-r weight leaves only the bf16 rounding of the factors
    rng = np.random.default_rng(4)
    wr = bf(rng.standard_normal((64, 4)) @ rng.standard_normal((4, 64)) * 0.1)
    dr = oracle.lowrank_decompose(wr, bf(np.ones(64)), 4)
    assert np.abs(dr["residual"]).max() < 2.0 ** -7 * np.abs(dr["w_hat"]).max()


def test_quantize_weight_hand_case_and_rounding():
    r = np.zeros((1, 64), np.float32)
    r[0, 0], r[0, 1], r[0, 2] = 0.7, -0.35, 0.05
    codes, scales = oracle.quantize_weight(0, r)
    s = np.float16(0.7 / 7)  # fp16(0.1) = 0.0999755859375
    assert scales[0, 0] == s.view(np.uint16)
    q = np.stack([codes[0] & 0xF, codes[0] >> 4], -1).reshape(-1).astype(int)
    q = np.where(q >= 8, q - 16, q)
    assert list(q[:4]) == [7, -4, 1, 0]  # 7.0017 -> 7; -3.5009 -> -4; 0.5001 -> 1
    rng = np.random.default_rng(5)
    rr = (rng.standard_normal((8, 256)) * 0.01).astype(np.float32)
    codes, scales = oracle.quantize_weight(0, rr)
    q = np.stack([codes & 0xF, codes >> 4], -1).reshape(8, -1).astype(int)
    q = np.where(q >= 8, q - 16, q)
    sc = np.repeat(scales.view(np.float16).astype(np.float64), 64, axis=1)
    assert np.all(np.abs(q * sc - rr) <= 0.5 * sc * (1 + 1e-6))


@pytest.mark.parametrize("prec", [0, 1])
def test_quantize_weight_matches_the_activation_quantizer(prec):
    # on bf16-representable inputs without smoothing both take the same steps
    rng = np.random.default_rng(6)
    xb = bf(rng.standard_normal((6, 128)) * 3.0)
    alpha = 0.01 if prec == 1 else 1.0
    c1, s1 = oracle.quantize_act(prec, xb, None, alpha=alpha)
    c2, s2 = oracle.quantize_weight(prec, f(xb).astype(np.float32), alpha=alpha)
    np.testing.assert_array_equal(c1, c2)
    np.testing.assert_array_equal(s1, s2)


def test_awq_quantize_hand_cases():
    w = np.zeros((3, 64))
    w[0, 0], w[0, 1] = -1.0, 2.0       # lo -1, hi 2: s = fp16(0.2), z = 5
    w[2, 0], w[2, 1] = 0.5, 1.0        # lo 0 (range holds 0): z = 0
    codes, scales, zeros = oracle.awq_quantize_weight(bf(w))
    q = np.stack([codes & 0xF, codes >> 4], -1).reshape(3, -1).astype(int)
    s = scales.view(np.float16).astype(np.float64)
    z = zeros.view(np.float16).astype(np.float64)
    assert s[0, 0] == np.float64(np.float16(0.2)) and z[0, 0] == 5
    assert list(q[0, :3]) == [0, 15, 5]
    assert s[1, 0] == 0 and z[1, 0] == 0 and np.all(q[1] == 0)        # all-zero group
    assert z[2, 0] == 0 and q[2, 1] == 15 and q[2, 0] == 8             # 0.5 / fp16(1/15) = 7.5 -> 8
    # dequantized error within half a step on random weights
    rng = np.random.default_rng(7)
    wr = bf(rng.standard_normal((4, 256)) * 0.02)
    codes, scales, zeros = oracle.awq_quantize_weight(wr)
    q = np.stack([codes & 0xF, codes >> 4], -1).reshape(4, -1).astype(np.float64)
    s = np.repeat(scales.view(np.float16).astype(np.float64), 64, axis=1)
    z = np.repeat(zeros.view(np.float16).astype(np.float64), 64, axis=1)
    assert np.all(np.abs((q - z) * s - f(wr)) <= 0.5 * s * (1 + 1e-3) + 1e-12)
