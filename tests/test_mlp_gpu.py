"""Parity of the fused MLP up-projection (svdq_w4a4_gemm_gelu_quant) with the
oracle, through the C ABI.

The kernel quantizes its own h = bf16(GELU(y)) with y accumulated in fp32,
while the oracle quantizes bf16 of the exact (double) GELU: the two h agree
except where a value lies within rounding distance of a bf16 boundary, so
codes and scales are unique only away from such boundaries.  The checks are:
  * scales: every group within 2^-6 relative of the oracle's (two bf16 steps
    of the group maximum), and at most 10% of groups different at all (the
    GEMM's fp32 y carries a relative error near 1e-3: see the integer-to-float
    step of the int4 GEMM, so a few % of group maxima round to the
    neighbouring bf16 value);
  * codes: every GPU code is a valid rounding of the oracle's smoothed value,
    |q s - xh| <= s/2 + 2^-6 |xh| (or clamped at -8 / 7 with xh beyond the
    end), and at most 1% of codes differ from the oracle's;
  * XL1: max |xl1 - ref| / max |ref| <= 1e-2 (its consumer, the down
    projection's low-rank product, rounds it to bf16; here it differs by the
    h values that round to a neighbouring bf16 number, and the fp32 atomics
    sum in any order);
  * the whole MLP (where the up-projection's K, the down projection's output
    width, is a multiple of 128): the down projection run by svdq_w4a4_gemm
    on the fused kernel's own codes, scales and XL1, against the oracle's
    down projection of those same three outputs, a unique result:
    max-abs-rel <= 1e-2 on every row compared.
"""
import numpy as np
import pytest
import torch

import oracle
import bit_w4a4_quantized_smooth_amd as sq
from bit_w4a4_quantized_smooth_amd import synth

pytestmark = pytest.mark.gpu


def dev(a, dtype=None):
    if a is None:
        return None
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.view(dtype)
    return t.cuda()


def b16(bits, dtype=torch.bfloat16):
    return None if bits is None else dev(np.asarray(bits, np.uint16).view(np.int16), dtype)


def unpack(codes):
    lo = (codes & 0xF).astype(np.int16)
    hi = (codes >> 4).astype(np.int16)
    q = np.stack([lo, hi], axis=-1).reshape(codes.shape[0], -1)
    return np.where(q >= 8, q - 16, q)


def run(case, rows=None):
    up, dn = case["up"], case["down"]
    codes, scales = oracle.quantize_act(0, up["x"], up["lam"])
    xl1 = oracle.lowrank_down(up["x"], up["l1t"]) if up["rank"] else None
    c, s, x = sq.w4a4_gemm_gelu_quant(dev(codes), b16(scales, torch.float16), dev(up["w_codes"]),
                                      b16(up["w_scales"], torch.float16), dev(xl1) if up["rank"] else None,
                                      b16(up["l2t"]) if up["rank"] else None, b16(up["bias"]), b16(dn["lam"]),
                                      b16(dn["l1t"]) if dn["rank"] else None)
    # the down projection on the fused outputs; its output width is the
    # up-projection's K, which the GEMM takes only in whole 128-column tiles
    y = None
    if up["K"] % 128 == 0:
        y = sq.w4a4_gemm(0, c, s, dev(dn["w_codes"]), b16(dn["w_scales"], torch.float16), x,
                         b16(dn["l2t"]) if dn["rank"] else None, b16(dn["bias"]))
    torch.cuda.synchronize()
    ref = oracle.mlp_up_gelu_quant(codes, scales, up["w_codes"], up["w_scales"], xl1, up["l2t"], up["bias"],
                                   dn["lam"], dn["l1t"] if dn["rank"] else np.zeros((0, up["N"]), np.uint16),
                                   rows=rows)
    sel = slice(None) if rows is None else np.asarray(rows)
    full = dict(codes=c.cpu().numpy(), scales=s.cpu().view(torch.int16).numpy().view(np.uint16),
                xl1=None if x is None else x.cpu().numpy())
    got = dict(codes=full["codes"][sel], scales=full["scales"][sel],
               xl1=None if x is None else full["xl1"][sel],
               y=None if y is None else y.cpu().view(torch.int16).numpy().view(np.uint16)[sel],
               rows=np.arange(c.shape[0]) if rows is None else np.asarray(rows), full=full)
    return got, ref


def check(case, got, ref):
    dn = case["down"]
    s_g = got["scales"].astype(np.uint16).view(np.float16).astype(np.float64)
    s_o = ref["scales"].view(np.float16).astype(np.float64)
    rel = np.abs(s_g - s_o) / np.maximum(s_o, 1e-30)
    q_g, q_o = unpack(got["codes"]), unpack(ref["codes"])
    print(f"[mlp] scales differing {np.mean(s_g != s_o):.3%} (max rel {rel.max():.3g}), "
          f"codes differing {np.mean(q_g != q_o):.4%}", flush=True)
    assert rel.max() <= 2.0 ** -6, f"scale off by {rel.max():.3g}"
    assert np.mean(s_g != s_o) <= 0.10, f"{np.mean(s_g != s_o):.3%} of scales differ"
    xh = ref["xh"].astype(np.float64)
    s_rep = np.repeat(s_g, 64, axis=1)
    err = np.abs(q_g * s_rep - xh)
    ok = err <= 0.5 * s_rep + 2.0 ** -6 * np.abs(xh) + 1e-30
    ok |= (q_g == 7) & (xh >= 7 * s_rep * (1 - 2.0 ** -6))
    ok |= (q_g == -8) & (xh <= -8 * s_rep * (1 - 2.0 ** -6))
    assert ok.all(), f"{np.sum(~ok)} codes are not a rounding of the oracle's value"
    assert np.mean(q_g != q_o) <= 0.01, f"{np.mean(q_g != q_o):.3%} of codes differ"
    if dn["rank"]:
        e = np.max(np.abs(got["xl1"] - ref["xl1"])) / max(np.max(np.abs(ref["xl1"])), 1e-30)
        assert e <= 1e-2, f"xl1 max-abs-rel {e:.3g}"
    if got["y"] is None:
        return
    # the down projection on the fused kernel's own outputs, against the oracle
    # evaluated on exactly those codes, scales and XL1 (a unique result)
    full, rows = got["full"], got["rows"]
    N = dn["N"]
    ri, ci = np.repeat(rows, N), np.tile(np.arange(N), rows.size)
    yd, _ = oracle.w4a4_linear(0, full["codes"], full["scales"], dn["w_codes"], dn["w_scales"],
                               full["xl1"] if dn["rank"] else None, dn["l2t"] if dn["rank"] else None, dn["bias"],
                               rows=ri, cols=ci)
    yd = yd.reshape(rows.size, N)
    yg = synth.bf16_bits_to_f64(got["y"])
    row_err = np.max(np.abs(yg - yd), axis=1) / np.max(np.abs(yd))
    print(f"[mlp] down projection on the fused outputs: max-abs-rel {row_err.max():.3g} over {rows.size} rows",
          flush=True)
    assert row_err.max() <= 1e-2, f"down projection max-abs-rel {row_err.max():.3g}"


SMALL = {
    "mlp_256x512x256_r16": lambda: synth.mlp_layer(3001, 256, 512, 256, 16),
    "mlp_ragged_200x768x384_r32": lambda: synth.mlp_layer(3002, 200, 768, 384, 32),
    "mlp_37x256x128_r0": lambda: synth.mlp_layer(3003, 37, 256, 128, 0),
    # odd group count (5): per-stage scale loads instead of four-stage blocks;
    # the down projection (320 output columns) is not run
    "mlp_ragged_70x384x320_r16": lambda: synth.mlp_layer(3004, 70, 384, 320, 16),
}


@pytest.mark.parametrize("name", sorted(SMALL))
def test_mlp_fused_small(name):
    print(f"[mlp] {name}", flush=True)
    case = SMALL[name]()
    got, ref = run(case)
    check(case, got, ref)


def test_mlp_fused_dit_size_sampled_rows():
    # 1024x1024 diffusion-transformer MLP: 4608 tokens, 3072 -> 12288 -> 3072, rank 32
    print("[mlp] dit 4608x12288x3072", flush=True)
    case = synth.mlp_layer(1002, 4608, 12288, 3072, 32)
    rows = np.concatenate([np.random.default_rng(5).choice(4608, 12, replace=False), [0, 4607]])
    got, ref = run(case, rows=rows)
    check(case, got, ref)
