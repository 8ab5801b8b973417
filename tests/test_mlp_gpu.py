"""Parity of the fused MLP up-projection (svdq_w4a4_gemm_gelu_quant) with the
oracle, through the C ABI.

The kernel quantizes its own h = bf16(GELU(y)) with y accumulated in fp32,
while the oracle quantizes bf16 of the exact (double) GELU: the two h agree
except where y's error moves GELU(y) across a bf16 rounding boundary, so
codes and scales are unique only away from such boundaries.  The checks:
  * scales: every group within 2^-6 relative of the oracle's (two bf16 steps
    of the group maximum);
  * codes: every GPU code a valid rounding of the oracle's smoothed value,
    |q s - xh| <= s/2 + 2^-6 |xh| (or clamped at -8 / 7 with xh beyond the
    end);
  * how many scales and codes may differ at all is derived per case from the
    error model of the int4 GEMM's fp32 y (see flip_model): per element, the
    probability that h changes its bf16 rounding, from its own accumulation
    noise and deterministic shifts; a scale may differ only where an element
    within 2^-6 of its group's maximum flips (expected E_s), a code only where
    its own h flips and one bf16 step of h reaches the code's rounding
    boundary (expected E_h), or where its group's scale changed.  Allowed:
    E + 5 sqrt(E) + 3 differences (a 5-sigma Poisson margin), codes also 64
    per group whose scale differs;
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
from scipy.stats import norm

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
    ref["up_codes"], ref["up_scales"], ref["up_xl1"] = codes, scales, xl1
    sel = slice(None) if rows is None else np.asarray(rows)
    full = dict(codes=c.cpu().numpy(), scales=s.cpu().view(torch.int16).numpy().view(np.uint16),
                xl1=None if x is None else x.cpu().numpy())
    got = dict(codes=full["codes"][sel], scales=full["scales"][sel],
               xl1=None if x is None else full["xl1"][sel],
               y=None if y is None else y.cpu().view(torch.int16).numpy().view(np.uint16)[sel],
               rows=np.arange(c.shape[0]) if rows is None else np.asarray(rows), full=full)
    return got, ref


C0 = float(np.array([0x3E22F983], np.uint32).view(np.float32)[0])  # the GEMM's accumulator seed
U = 2.0 ** -24  # half an ulp of fp32, relative


def flip_model(case, rows, ref):
    """Per h element, the probability that the kernel's bf16(GELU(y)) differs
    from the oracle's bf16(GELU(y)), from an error model of the kernel's y:
      * noise: each group adds S_g (c0 + P_g 2^-18) to an fp32 accumulator
        whose magnitude is about c0 T_t (T_t = sum of the first t scale
        products S = sa sw), so its rounding is uniform within half an ulp,
        standard deviation 2^-24 c0 T_t / sqrt 3, times 2^18 in y; plus the
        removal of c0 sum S in 32-group chunks (the matrix instruction's 31
        fp32 additions of each chunk and one subtraction);
      * a deterministic shift: XL1 rounded to bf16 before the low-rank
        product;
      * a bounded part: fp32 rounding of the low-rank product, bias and GELU
        (a few ulp) and the GELU approximation (|erf error| < 1.5e-7).
    h is GELU(y) shifted by GELU'(y) times the y error; it flips where the
    shift crosses either end of its bf16 rounding cell."""
    up = case["up"]
    sa = oracle.f16_to_f32(ref["up_scales"][rows]).astype(np.float64)         # [R, G]
    sw = oracle.f16_to_f32(up["w_scales"]).astype(np.float64)                 # [N, G]
    S = sa[:, None, :] * sw[None, :, :]                                       # [R, N, G]
    T = np.cumsum(S, axis=2)
    var = (2.0 ** 18 * U * C0) ** 2 / 3.0 * np.sum(T * T, axis=2)
    G = S.shape[2]
    for c in range(0, G, 32):
        Tc = S[:, :, c:c + 32].sum(axis=2)
        Trem = T[:, :, -1] - T[:, :, min(c + 32, G) - 1]
        var += (2.0 ** 18 * U * C0) ** 2 / 3.0 * (31.0 * Tc * Tc + Trem * Trem)
    sigma = np.sqrt(var)
    y = ref["y"]                                                               # [R, N] double
    slack = np.zeros_like(y)
    shift = np.zeros_like(y)
    if up["rank"]:
        xl1 = ref["up_xl1"][rows].astype(np.float64)                           # [R, r]
        xl1b = synth.bf16_bits_to_f64(oracle.f32_to_bf16(ref["up_xl1"][rows].astype(np.float32)))
        l2 = synth.bf16_bits_to_f64(up["l2t"])                                 # [N, r]
        shift = (xl1b - xl1) @ l2.T
        slack += U * (up["rank"] + 2) * (np.abs(xl1b) @ np.abs(l2).T)
    h, _ = oracle.gelu(y)
    slack += U * 4 * np.abs(y)
    dg = norm.cdf(y) + y * norm.pdf(y)                                         # GELU'(y)
    hslack = np.abs(dg) * slack + 0.5 * np.abs(y) * 1.5e-7 + 8 * U * np.abs(h)
    mu, sd = dg * shift, np.abs(dg) * sigma + 1e-300
    # the bf16 rounding cell of h (the reals that round to the oracle's bf16 h):
    # half a step on either side, the step below a power of two being half
    hb = synth.bf16_bits_to_f64(ref["h_bf16"])
    a = np.abs(hb)
    m, e = np.frexp(a)                                                         # a = m 2^e, m in [0.5, 1)
    step = np.maximum(np.ldexp(1.0, e - 8), 2.0 ** -133)                       # 8 significant bits
    below = np.where(m == 0.5, step / 2, step)
    top, bottom = a + step / 2, a - below / 2                                  # the cell of |h|
    hi = np.where(hb >= 0, top, -bottom) - h
    lo = h - np.where(hb >= 0, bottom, -top)
    p = norm.sf((np.maximum(hi - hslack, 0) - mu) / sd) + norm.cdf((-np.maximum(lo - hslack, 0) - mu) / sd)
    return np.minimum(p, 1.0)


def allowance(e):
    return e + 5.0 * np.sqrt(e) + 3.0


def check(case, got, ref):
    dn = case["down"]
    rows = got["rows"]
    s_g = got["scales"].astype(np.uint16).view(np.float16).astype(np.float64)
    s_o = ref["scales"].view(np.float16).astype(np.float64)
    rel = np.abs(s_g - s_o) / np.maximum(s_o, 1e-30)
    q_g, q_o = unpack(got["codes"]), unpack(ref["codes"])
    # derived allowances for the number of differing scales and codes
    p = flip_model(case, rows, ref)                                            # [R, N]
    xh = ref["xh"].astype(np.float64)
    R, N = xh.shape
    ax = np.abs(xh).reshape(R, N // 64, 64)
    near_max = ax >= ax.max(axis=2, keepdims=True) * (1 - 2.0 ** -6)
    e_s = float(np.minimum(1.0, np.sum(p.reshape(R, N // 64, 64) * near_max, axis=2)).sum())
    # a flip moves xh by at most one bf16 step of h times 1/lambda (and the fp32
    # rounding of the product): the code can change only where its rounding
    # boundary (q +- 1/2) s lies that close to xh
    so = np.repeat(s_o, 64, axis=1)
    inv_lam = (1.0 / synth.bf16_bits_to_f64(dn["lam"]))[None, :]
    hstep = np.ldexp(1.0, np.frexp(np.abs(synth.bf16_bits_to_f64(ref["h_bf16"])))[1] - 8)
    t = xh / so
    bdist = so * np.minimum(np.abs(t - (q_o + 0.5)), np.abs(t - (q_o - 0.5)))
    reach = bdist <= 1.01 * hstep * inv_lam + 2.0 ** -20 * np.abs(xh)
    e_h = float(np.sum(p * reach))
    d_s, d_c = int(np.sum(s_g != s_o)), int(np.sum(q_g != q_o))
    print(f"[mlp] scales differing {d_s} of {s_g.size} (expected <= {e_s:.1f}, max rel {rel.max():.3g}); "
          f"codes differing {d_c} of {q_g.size} (expected <= {e_h:.1f} from h flips near a code boundary, "
          f"{float(p.sum()):.0f} h flips in all)", flush=True)
    assert rel.max() <= 2.0 ** -6, f"scale off by {rel.max():.3g}"
    assert d_s <= allowance(e_s), f"{d_s} scales differ; the error model allows {allowance(e_s):.1f}"
    assert d_c <= allowance(e_h) + 64 * d_s, f"{d_c} codes differ; the error model allows {allowance(e_h) + 64 * d_s:.1f}"
    s_rep = np.repeat(s_g, 64, axis=1)
    err = np.abs(q_g * s_rep - xh)
    ok = err <= 0.5 * s_rep + 2.0 ** -6 * np.abs(xh) + 1e-30
    ok |= (q_g == 7) & (xh >= 7 * s_rep * (1 - 2.0 ** -6))
    ok |= (q_g == -8) & (xh <= -8 * s_rep * (1 - 2.0 ** -6))
    assert ok.all(), f"{np.sum(~ok)} codes are not a rounding of the oracle's value"
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
