"""Parity of the fused attention projection (svdq_w4a4_gemm_qkv_norm_rope) with
the oracle, through the C ABI.

The GEMM inputs are the oracle's own activation codes, scales and XL1, so this
checks the GEMM + epilogue alone.  Bar: each of the Q, K and V column blocks
within 1e-2 max-abs-rel of the oracle's double result before bf16 rounding
(max |Y_gpu - y| / max |y| over the block; Q and K are compared after the
norm, whose outputs are O(norm weight)).  Small workloads are compared in
full; the diffusion-transformer size on whole sampled token rows (every
column, so every head is checked whole).  The V block must also equal the
plain GEMM's output bit for bit (same accumulation, same rounding).
"""
import numpy as np
import pytest
import torch

import oracle
import bit_w4a4_quantized_smooth_amd as sq
from bit_w4a4_quantized_smooth_amd import synth

pytestmark = pytest.mark.gpu

TOL = 1e-2


def dev(a, dtype=None):
    if a is None:
        return None
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.view(dtype)
    return t.cuda()


def bf16_dev(bits):
    return None if bits is None else dev(np.asarray(bits, np.uint16).view(np.int16), torch.bfloat16)


def scales_dev(prec, s):
    return dev(np.asarray(s, np.uint16).view(np.int16), torch.float16) if prec == sq.SVDQ_INT4 else dev(s)


def host_bits(t):
    return t.cpu().view(torch.int16).numpy().view(np.uint16)


def oracle_inputs(d):
    codes, scales = oracle.quantize_act(d["prec"], d["x"], d["lam"], alpha=d["alpha_a"])
    xl1 = oracle.lowrank_down(d["x"], d["l1t"]) if d["rank"] else None
    return codes, scales, xl1


def run_fused(d, codes, scales, xl1):
    y = sq.w4a4_gemm_qkv_norm_rope(
        d["prec"], dev(codes), scales_dev(d["prec"], scales), dev(d["w_codes"]),
        scales_dev(d["prec"], d["w_scales"]), dev(xl1) if d["rank"] else None,
        bf16_dev(d["l2t"]) if d["rank"] else None, bf16_dev(d["bias"]), d["heads"], d["head_dim"],
        bf16_dev(d["norm_q"]), bf16_dev(d["norm_k"]), d["eps"], dev(d["rope"]), d["alpha_a"], d["alpha_w"])
    torch.cuda.synchronize()
    return host_bits(y)


def run_plain(d, codes, scales, xl1):
    y = sq.w4a4_gemm(d["prec"], dev(codes), scales_dev(d["prec"], scales), dev(d["w_codes"]),
                     scales_dev(d["prec"], d["w_scales"]), dev(xl1) if d["rank"] else None,
                     bf16_dev(d["l2t"]) if d["rank"] else None, bf16_dev(d["bias"]), d["alpha_a"], d["alpha_w"])
    torch.cuda.synchronize()
    return host_bits(y)


def check_blocks(y_bits, ref, HD):
    got = synth.bf16_bits_to_f64(y_bits)
    for b, name in enumerate("QKV"):
        g, r = got[:, b * HD:(b + 1) * HD], ref[:, b * HD:(b + 1) * HD]
        err = np.max(np.abs(g - r)) / max(np.max(np.abs(r)), 1e-30)
        assert err <= TOL, f"{name} block: max-abs-rel {err:.3g}"


SMALL = {
    "int4_d128_h2_256x512_r16": lambda: synth.qkv_layer(2001, 256, 2, 128, 512, 16, synth.INT4),
    "int4_d64_h4_ragged200x320_r32": lambda: synth.qkv_layer(2002, 200, 4, 64, 320, 32, synth.INT4),
    "int4_d128_h1x3_batch2_r0_nobias": lambda: synth.qkv_layer(2003, 2 * 96, 2, 128, 256, 0, synth.INT4,
                                                               S=96, with_bias=False),
    "int4_d128_h2_norope_130x256_r16": lambda: synth.qkv_layer(2004, 130, 2, 128, 256, 16, synth.INT4,
                                                               with_rope=False),
    "nvfp4_d128_h2_256x512_r32": lambda: synth.qkv_layer(2005, 256, 2, 128, 512, 32, synth.NVFP4),
    "nvfp4_d64_h2_ragged37x768_r16": lambda: synth.qkv_layer(2006, 37, 2, 64, 768, 16, synth.NVFP4),
    "nvfp4_d128_h4_batch3_r16": lambda: synth.qkv_layer(2007, 3 * 64, 4, 128, 256, 16, synth.NVFP4, S=64),
    "nvfp4_d64_h2_ragged50x448_r16": lambda: synth.qkv_layer(2008, 50, 2, 64, 448, 16, synth.NVFP4),
}


@pytest.mark.parametrize("name", sorted(SMALL))
def test_qkv_small(name):
    print(f"[qkv] {name}", flush=True)
    d = SMALL[name]()
    codes, scales, xl1 = oracle_inputs(d)
    y = run_fused(d, codes, scales, xl1)
    ref, _ = oracle.w4a4_linear_qkv(d["prec"], codes, scales, d["w_codes"], d["w_scales"], xl1, d["l2t"],
                                    d["bias"], d["heads"], d["head_dim"], d["norm_q"], d["norm_k"], d["eps"],
                                    d["rope"], d["alpha_a"], d["alpha_w"])
    HD = d["heads"] * d["head_dim"]
    check_blocks(y, ref, HD)
    plain = run_plain(d, codes, scales, xl1)
    M, K = d["x"].shape
    tiles = -(-M // 128) * (3 * HD // 128)
    if d["prec"] == sq.SVDQ_INT4 and K % 256 == 0 and tiles <= torch.cuda.get_device_properties(0).multi_processor_count:
        # a plain int4 GEMM of at most one tile per CU runs on the K-split
        # kernel (the two halves of K summed in another fp32 order)
        g, r = synth.bf16_bits_to_f64(y[:, 2 * HD:]), synth.bf16_bits_to_f64(plain[:, 2 * HD:])
        assert np.max(np.abs(g - r)) <= TOL * max(np.max(np.abs(r)), 1e-30), "V block vs the plain GEMM"
    else:
        assert np.array_equal(y[:, 2 * HD:], plain[:, 2 * HD:]), "V block differs from the plain GEMM"


@pytest.mark.parametrize("prec", [sq.SVDQ_INT4, sq.SVDQ_NVFP4])
def test_qkv_dit_size_sampled_rows(prec):
    # 1024x1024 diffusion-transformer attention: 4608 tokens, 24 heads of 128, hidden 3072
    print(f"[qkv] dit 4608x9216x3072 prec {prec}", flush=True)
    d = synth.qkv_layer(1002 if prec == sq.SVDQ_INT4 else 1004, 4608, 24, 128, 3072, 32, prec, 0.005, 30.0)
    codes, scales, xl1 = oracle_inputs(d)
    y = run_fused(d, codes, scales, xl1)
    rows = np.concatenate([np.random.default_rng(7).choice(4608, 20, replace=False), [0, 127, 4480, 4607]])
    ref, _ = oracle.w4a4_linear_qkv(d["prec"], codes, scales, d["w_codes"], d["w_scales"], xl1, d["l2t"],
                                    d["bias"], d["heads"], d["head_dim"], d["norm_q"], d["norm_k"], d["eps"],
                                    d["rope"], d["alpha_a"], d["alpha_w"], rows=rows)
    check_blocks(y[rows], ref, 24 * 128)


def test_qkv_empty():
    d = synth.qkv_layer(2008, 0, 2, 128, 256, 16, synth.INT4)
    y = sq.w4a4_gemm_qkv_norm_rope(0, torch.empty((0, 128), dtype=torch.uint8, device="cuda"),
                                   torch.empty((0, 4), dtype=torch.float16, device="cuda"), dev(d["w_codes"]),
                                   scales_dev(0, d["w_scales"]), torch.empty((0, 16), device="cuda"),
                                   bf16_dev(d["l2t"]), None, 2, 128, bf16_dev(d["norm_q"]), bf16_dev(d["norm_k"]),
                                   1e-6, dev(d["rope"]))
    torch.cuda.synchronize()
    assert y.shape == (0, 768)
