"""Pins of the oracle's Q/K/V epilogue (per-head RMSNorm of Q and K, then the
rotary embedding; V untouched) against closed forms and hand-worked values,
each chosen so that a plausible slip fails: eps inside vs outside the root,
swapped norm weights, weights indexed by column instead of by channel, head
boundaries, the sign of the sine term, adjacent-pair vs half-split pairing,
and the table row used by each token.
"""
import numpy as np
import pytest

import oracle


def bf16_const(v, n):
    import struct
    b = struct.unpack("<I", struct.pack("<f", float(v)))[0] >> 16
    return np.full(n, b, np.uint16)


def bf16_vec(vals):
    import struct
    return np.array([struct.unpack("<I", struct.pack("<f", float(v)))[0] >> 16 for v in vals], np.uint16)


def ones(D):
    return bf16_const(1.0, D)


def test_unit_rms_and_v_untouched():
    rng = np.random.default_rng(0)
    H, D = 3, 64
    y = rng.standard_normal((5, 3 * H * D)) * rng.uniform(0.1, 50, size=(5, 1))
    out, _ = oracle.qkv_norm_rope(y, None, H, D, ones(D), ones(D), 0.0)
    heads = out[:, :2 * H * D].reshape(5, 2 * H, D)
    np.testing.assert_allclose(np.mean(heads ** 2, axis=2), 1.0, rtol=1e-12)
    assert np.array_equal(out[:, 2 * H * D:], y[:, 2 * H * D:])
    # direction of each head is kept (a positive multiple of the input head)
    yin = y[:, :2 * H * D].reshape(5, 2 * H, D)
    ratio = heads / yin
    np.testing.assert_allclose(ratio, ratio[:, :, :1].repeat(D, axis=2), rtol=1e-12)
    assert np.all(ratio > 0)


def test_q_and_k_weights_not_swapped():
    rng = np.random.default_rng(1)
    H, D = 2, 64
    y = rng.standard_normal((4, 3 * H * D))
    out, _ = oracle.qkv_norm_rope(y, None, H, D, bf16_const(2.0, D), bf16_const(3.0, D), 0.0)
    rms = np.sqrt(np.mean(out[:, :2 * H * D].reshape(4, 2 * H, D) ** 2, axis=2))
    np.testing.assert_allclose(rms[:, :H], 2.0, rtol=1e-12)
    np.testing.assert_allclose(rms[:, H:], 3.0, rtol=1e-12)


def test_scale_invariance_without_eps():
    rng = np.random.default_rng(2)
    H, D = 2, 128
    y = rng.standard_normal((3, 3 * H * D))
    w = bf16_vec(rng.uniform(0.5, 2.0, D))
    a, _ = oracle.qkv_norm_rope(y, None, H, D, w, w, 0.0)
    b, _ = oracle.qkv_norm_rope(1000.0 * y, None, H, D, w, w, 0.0)
    np.testing.assert_allclose(a[:, :2 * H * D], b[:, :2 * H * D], rtol=1e-12)
    np.testing.assert_allclose(b[:, 2 * H * D:], 1000.0 * y[:, 2 * H * D:], rtol=0)


@pytest.mark.parametrize("a,eps", [(0.5, 1e-6), (1e-3, 1e-6), (2.0, 0.25), (0.0, 1e-6)])
def test_constant_head_closed_form(a, eps):
    # a head whose entries all equal a: mean square a^2, so every output is a / sqrt(a^2 + eps)
    H, D = 1, 64
    y = np.full((1, 3 * H * D), a)
    out, _ = oracle.qkv_norm_rope(y, None, H, D, ones(D), ones(D), eps)
    np.testing.assert_allclose(out[0, :2 * D], a / np.sqrt(a * a + eps), rtol=1e-14)


def test_weights_indexed_by_channel_within_head():
    # constant heads normalize to exactly w_d, in every head of Q and of K
    H, D = 3, 64
    y = np.repeat(np.array([[0.3, 5.0, 70.0, 0.01, 2.0, 9.0, 1.0, 1.0, 1.0]]), D, axis=1).reshape(1, 9 * D)
    wq = bf16_vec(np.arange(1, D + 1) / 8.0)
    wk = bf16_vec(-np.arange(1, D + 1) / 16.0)
    out, _ = oracle.qkv_norm_rope(y, None, H, D, wq, wk, 0.0)
    for h in range(H):
        np.testing.assert_allclose(out[0, h * D:(h + 1) * D], np.arange(1, D + 1) / 8.0, rtol=1e-14)
        np.testing.assert_allclose(out[0, (H + h) * D:(H + h + 1) * D], -np.arange(1, D + 1) / 16.0, rtol=1e-14)
    np.testing.assert_array_equal(out[0, 2 * H * D:], y[0, 2 * H * D:])


def _unit_head_rows(D, H, first=(8.0, 0.0)):
    # every Q/K head is 8 * e_0 (mean square 1: the norm leaves it as it is)
    y = np.zeros((1, 3 * H * D))
    for h in range(2 * H):
        y[0, h * D] = first[0]
        y[0, h * D + 1] = first[1]
    return y


def test_rotary_pairs_are_adjacent_and_sine_sign():
    H, D = 1, 64
    # head = 8 e_0: rotating pair 0 by +90 degrees (cos 0, sin 1) moves it to channel 1 as +8;
    # a half-split pairing would move it to channel D/2 instead
    rope = np.zeros((1, D // 2, 2), np.float32)
    rope[..., 0] = 1.0
    rope[0, 0] = (0.0, 1.0)
    out, _ = oracle.qkv_norm_rope(_unit_head_rows(D, H), None, H, D, ones(D), ones(D), 0.0, rope)
    for h in range(2 * H):
        expect = np.zeros(D)
        expect[1] = 8.0
        np.testing.assert_allclose(out[0, h * D:(h + 1) * D], expect, atol=1e-14)
    # worked example: pair 0 = (a, b) = (6, 2 sqrt 7), mean square of the head 1;
    # rotated by -90 degrees (cos 0, sin -1) -> (b, -a), by 180 degrees -> (-a, -b)
    b = 2.0 * np.sqrt(7.0)
    y = _unit_head_rows(D, H, first=(6.0, b))
    rope[0, 0] = (0.0, -1.0)
    out, _ = oracle.qkv_norm_rope(y, None, H, D, ones(D), ones(D), 0.0, rope)
    np.testing.assert_allclose(out[0, :2], [b, -6.0], rtol=1e-14)
    rope[0, 0] = (-1.0, 0.0)
    out, _ = oracle.qkv_norm_rope(y, None, H, D, ones(D), ones(D), 0.0, rope)
    np.testing.assert_allclose(out[0, :2], [-6.0, -b], rtol=1e-14)


def test_rotation_keeps_pair_norms_and_uses_token_row_mod_s():
    rng = np.random.default_rng(3)
    H, D, S = 2, 128, 3
    y = rng.standard_normal((7, 3 * H * D))
    theta = rng.uniform(-np.pi, np.pi, (S, D // 2))
    rope = np.stack([np.cos(theta), np.sin(theta)], axis=-1).astype(np.float32)
    plain, _ = oracle.qkv_norm_rope(y, np.arange(7), H, D, ones(D), ones(D), 1e-6)
    rot, _ = oracle.qkv_norm_rope(y, np.arange(7), H, D, ones(D), ones(D), 1e-6, rope)
    P = plain[:, :2 * H * D].reshape(7, 2 * H, D // 2, 2)
    R = rot[:, :2 * H * D].reshape(7, 2 * H, D // 2, 2)
    np.testing.assert_allclose(np.hypot(R[..., 0], R[..., 1]), np.hypot(P[..., 0], P[..., 1]), rtol=1e-6)
    # rotation angle of each pair equals the table angle of row m mod S
    ang = np.angle((R[..., 0] + 1j * R[..., 1]) / (P[..., 0] + 1j * P[..., 1]))
    for m in range(7):
        d = np.angle(np.exp(1j * (ang[m] - theta[m % S][None, :])))
        assert np.max(np.abs(d)) < 1e-5
    # the row ids, not the position in y, pick the table row
    rot2, _ = oracle.qkv_norm_rope(y[3:4], np.array([3]), H, D, ones(D), ones(D), 1e-6, rope)
    np.testing.assert_array_equal(rot2[0], rot[3])


def test_norm_weight_applies_before_rotation():
    # head 8 e_0, w_0 = 2, other weights 1: the norm gives 16 e_0, the +90 degree
    # rotation of pair 0 then gives 16 e_1 (rotating first would give 8 e_1)
    H, D = 1, 64
    w = ones(D)
    w[0] = bf16_const(2.0, 1)[0]
    rope = np.zeros((1, D // 2, 2), np.float32)
    rope[..., 0] = 1.0
    rope[0, 0] = (0.0, 1.0)
    out, _ = oracle.qkv_norm_rope(_unit_head_rows(D, H), None, H, D, w, w, 0.0, rope)
    np.testing.assert_allclose(out[0, :2], [0.0, 16.0], atol=1e-14)


def test_linear_qkv_composes_linear_and_epilogue():
    from bit_w4a4_quantized_smooth_amd import synth
    H, D = 1, 64
    d = synth.svdq_layer(5, 6, 3 * H * D, 128, 16, synth.INT4, 0.01, 20.0)
    codes, scales = oracle.quantize_act(d["prec"], d["x"], d["lam"])
    xl1 = oracle.lowrank_down(d["x"], d["l1t"])
    y, _ = oracle.w4a4_linear(d["prec"], codes, scales, d["w_codes"], d["w_scales"], xl1, d["l2t"], d["bias"])
    w = bf16_vec(np.linspace(0.5, 1.5, D))
    full, _ = oracle.w4a4_linear_qkv(d["prec"], codes, scales, d["w_codes"], d["w_scales"], xl1, d["l2t"],
                                     d["bias"], H, D, w, w, 1e-6)
    ref, _ = oracle.qkv_norm_rope(y, None, H, D, w, w, 1e-6)
    np.testing.assert_array_equal(full, ref)
    some, _ = oracle.w4a4_linear_qkv(d["prec"], codes, scales, d["w_codes"], d["w_scales"], xl1, d["l2t"],
                                     d["bias"], H, D, w, w, 1e-6, rows=[4, 1])
    np.testing.assert_array_equal(some, ref[[4, 1]])
