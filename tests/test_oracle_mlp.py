"""Pins of the oracle's MLP pieces: GELU (erf form) against normal-table values
and exact identities, the smoothing step against exact cases, and the fused
up-projection composition (linear -> GELU -> bf16 -> quantize + X.L1) against
its separately pinned parts."""
import numpy as np
import pytest

import oracle
from bit_w4a4_quantized_smooth_amd import synth


def test_gelu_normal_table_values():
    # GELU(y) = y * Phi(y); Phi from standard normal tables
    y = np.array([0.0, 1.0, 2.0, -1.0, 1.96, -1.96, 3.0])
    phi = np.array([0.5, 0.8413447461, 0.9772498681, 0.1586552539, 0.9750021049, 0.0249978951, 0.9986501020])
    h, _ = oracle.gelu(y)
    np.testing.assert_allclose(h, y * phi, rtol=0, atol=1e-9)  # tables to 10 decimals


def test_gelu_identities():
    rng = np.random.default_rng(0)
    y = np.concatenate([rng.standard_normal(1000) * 3, [1e-8, 5.0, 8.0, 12.0]])
    hp, _ = oracle.gelu(y)
    hn, _ = oracle.gelu(-y)
    # y Phi(y) - (-y) Phi(-y) = y (Phi(y) + Phi(-y)) = y
    np.testing.assert_allclose(hp - hn, y, rtol=1e-13, atol=1e-15)
    # far tails: GELU(y) -> y, GELU(-y) -> tiny negative (not a cancelled zero)
    big, _ = oracle.gelu(np.array([10.0, -10.0]))
    assert big[0] == 10.0
    assert -1e-22 < big[1] < -1e-23
    # global minimum near y = -0.7518 with value about -0.16997
    g = np.linspace(-2, 0, 20001)
    hg, _ = oracle.gelu(g)
    assert abs(g[np.argmin(hg)] + 0.7518) < 1e-3 and abs(hg.min() + 0.16997) < 1e-4


def test_gelu_bf16_rounding():
    # values exactly representable in bf16 stay; the large-y tail is y itself
    y = np.array([16.0, 24.0, -0.0])
    _, hb = oracle.gelu(y)
    assert list(hb) == [0x4180, 0x41C0, 0x8000]
    # ties round to the even mantissa (bf16 spacing is 2 at 256): 257 -> 256, 259 -> 260
    _, hb2 = oracle.gelu(np.array([257.0, 259.0]))
    assert list(hb2) == [0x4380, 0x4382]


def test_smooth_exact_cases():
    rng = np.random.default_rng(1)
    x = synth.to_bf16_bits(rng.standard_normal((3, 128)))
    xf = synth.bf16_bits_to_f64(x)
    np.testing.assert_array_equal(oracle.smooth(x, None), xf.astype(np.float32))
    lam2 = synth.to_bf16_bits(np.full(128, 2.0))
    np.testing.assert_array_equal(oracle.smooth(x, lam2), (xf / 2).astype(np.float32))


def test_mlp_up_composition():
    d = synth.svdq_layer(11, 8, 256, 128, 16, synth.INT4, 0.01, 20.0)
    codes, scales = oracle.quantize_act(0, d["x"], d["lam"])
    xl1 = oracle.lowrank_down(d["x"], d["l1t"])
    rng = np.random.default_rng(2)
    lam_down = synth.to_bf16_bits(rng.uniform(0.5, 2.0, 256))
    l1t_down = synth.to_bf16_bits(rng.normal(0, 0.02, (16, 256)))
    out = oracle.mlp_up_gelu_quant(codes, scales, d["w_codes"], d["w_scales"], xl1, d["l2t"], d["bias"],
                                   lam_down, l1t_down)
    y, _ = oracle.w4a4_linear(0, codes, scales, d["w_codes"], d["w_scales"], xl1, d["l2t"], d["bias"])
    np.testing.assert_array_equal(out["y"], y)
    _, hb = oracle.gelu(y)
    np.testing.assert_array_equal(out["h_bf16"], hb)
    c2, s2 = oracle.quantize_act(0, hb, lam_down)
    np.testing.assert_array_equal(out["codes"], c2)
    np.testing.assert_array_equal(out["scales"], s2)
    np.testing.assert_array_equal(out["xl1"], oracle.lowrank_down(hb, l1t_down))
    some = oracle.mlp_up_gelu_quant(codes, scales, d["w_codes"], d["w_scales"], xl1, d["l2t"], d["bias"],
                                    lam_down, l1t_down, rows=[5, 2])
    np.testing.assert_array_equal(some["codes"], out["codes"][[5, 2]])
    np.testing.assert_array_equal(some["xl1"], out["xl1"][[5, 2]])


def test_mlp_up_composition_nvfp4():
    # the nvfp4 form: the up projection with its global scales, then the down
    # projection's nvfp4 quantization of h with its own global scale
    d = synth.svdq_layer(12, 8, 256, 128, 16, synth.NVFP4, 0.01, 20.0)
    codes, scales = oracle.quantize_act(1, d["x"], d["lam"], alpha=d["alpha_a"])
    xl1 = oracle.lowrank_down(d["x"], d["l1t"])
    rng = np.random.default_rng(3)
    lam_down = synth.to_bf16_bits(rng.uniform(0.5, 2.0, 256))
    l1t_down = synth.to_bf16_bits(rng.normal(0, 0.02, (16, 256)))
    ao = 2.0 ** -6
    kw = dict(prec=1, alpha_a=d["alpha_a"], alpha_w=d["alpha_w"], alpha_out=ao)
    out = oracle.mlp_up_gelu_quant(codes, scales, d["w_codes"], d["w_scales"], xl1, d["l2t"], d["bias"],
                                   lam_down, l1t_down, **kw)
    y, _ = oracle.w4a4_linear(1, codes, scales, d["w_codes"], d["w_scales"], xl1, d["l2t"], d["bias"],
                              alpha_a=d["alpha_a"], alpha_w=d["alpha_w"])
    np.testing.assert_array_equal(out["y"], y)
    _, hb = oracle.gelu(y)
    np.testing.assert_array_equal(out["h_bf16"], hb)
    c2, s2 = oracle.quantize_act(1, hb, lam_down, alpha=ao)
    assert out["scales"].dtype == np.uint8 and out["scales"].shape == (8, 256 // 16)
    np.testing.assert_array_equal(out["codes"], c2)
    np.testing.assert_array_equal(out["scales"], s2)
    np.testing.assert_array_equal(out["xl1"], oracle.lowrank_down(hb, l1t_down))
    # every code decodes to within half an E2M1 step of xh / (s alpha) (E2M1
    # steps 0.5 / 1 / 2 above 0 / 2 / 4), or saturates at 6
    s = oracle.e4m3_to_f32(out["scales"]).astype(np.float64)
    lo, hi = out["codes"] & 0xF, out["codes"] >> 4
    q = np.stack([lo, hi], -1).reshape(8, 256)
    v = oracle.e2m1_to_f32(q).astype(np.float64)
    t = out["xh"].astype(np.float64) / (np.repeat(s, 16, axis=1) * ao)
    half = np.where(np.abs(v) < 2, 0.25, np.where(np.abs(v) < 4, 0.5, 1.0))
    assert np.all((np.abs(v - t) <= half * (1 + 1e-6)) | ((np.abs(v) == 6) & (np.abs(t) >= 5)))
    some = oracle.mlp_up_gelu_quant(codes, scales, d["w_codes"], d["w_scales"], xl1, d["l2t"], d["bias"],
                                    lam_down, l1t_down, rows=[6, 1], **kw)
    np.testing.assert_array_equal(some["codes"], out["codes"][[6, 1]])
    np.testing.assert_array_equal(some["scales"], out["scales"][[6, 1]])


@pytest.mark.parametrize("prec", [synth.INT4, synth.NVFP4])
def test_mlp_layer_generator(prec):
    # shapes, dtypes and format of the synthetic MLP pair in both precisions
    case = synth.mlp_layer(5, 20, 256, 128, 16, prec)
    up, dn = case["up"], case["down"]
    G = 64 if prec == synth.INT4 else 16
    assert up["N"] == 256 and up["K"] == 128 and dn["N"] == 128 and dn["K"] == 256
    assert dn["w_codes"].shape == (128, 128) and dn["w_codes"].dtype == np.uint8
    assert dn["w_scales"].shape == (128, 256 // G)
    assert dn["w_scales"].dtype == (np.uint16 if prec == synth.INT4 else np.uint8)
    assert dn["l1t"].shape == (16, 256) and dn["l2t"].shape == (128, 16) and dn["lam"].shape == (256,)
    if prec == synth.NVFP4:
        assert dn["alpha_a"] == 2.0 ** -6 and dn["alpha_w"] == 2.0 ** -6
        sw = oracle.e4m3_to_f32(dn["w_scales"]).astype(np.float64) * dn["alpha_w"]
        assert np.all((sw >= 0.005 * (1 - 2 ** -4)) & (sw <= 0.02 * (1 + 2 ** -4)))  # one E4M3 rounding
    else:
        assert dn["alpha_a"] == 1.0 and dn["alpha_w"] == 1.0
