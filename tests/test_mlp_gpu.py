"""Parity of the fused MLP up-projection (svdq_w4a4_gemm_gelu_quant) with the
oracle, through the C ABI, in both precisions (int4 g64 with fp16 scales,
nvfp4 g16 with E4M3 scales and global scales).

The kernel quantizes its own h = bf16(GELU(y)) with y accumulated in fp32,
while the oracle quantizes bf16 of the exact (double) GELU: the two h agree
except where y's error moves GELU(y) across a bf16 rounding boundary, so
codes and scales are unique only away from such boundaries.  The checks:
  * scales: every group's scale one the kernel may have written: its amax
    between the bounds of |xh| that the error model below gives
    (xh_interval), through the scale's rounding (int4 fp16 of amax / 7,
    nvfp4 E4M3 of amax / (6 alpha)) (scale_range);
  * codes: every GPU code a valid rounding, with the GPU's own scale s, of
    some t = xh / (s alpha) (alpha = 1 for int4) the kernel may have
    quantized: the oracle's y widened by the error model's bound on the
    kernel's y error, through GELU, the bf16 rounding of h and 1/lambda
    (t_interval); int4 grid -8..7, nvfp4 the E2M1 magnitudes with t's sign
    (kept at zero, so either sign where the interval spans 0; +0 and -0
    count as equal codes);
  * how many scales and codes may differ at all is derived per case from the
    error model of the GEMM's fp32 y (see flip_model): per element, the
    probability that h changes its bf16 rounding, from its own accumulation
    noise and deterministic shifts; a scale may differ only where an element
    within 2^-6 of its group's maximum flips (expected E_s; nvfp4: and the
    scale's argument amax / (6 alpha) lies within 2^-7 of an E4M3 rounding
    boundary), a code only where its own h flips and one bf16 step of h
    reaches the code's rounding boundary (expected E_h), or where its group's
    scale changed.  Allowed: E + 5 sqrt(E) + 3 differences (a 5-sigma Poisson
    margin), codes also a whole group (64 int4 or 16 nvfp4 codes) per group
    whose scale differs;
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
from scipy.optimize import brentq
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


def nibbles(codes):
    lo = (codes & 0xF).astype(np.int16)
    hi = (codes >> 4).astype(np.int16)
    return np.stack([lo, hi], axis=-1).reshape(codes.shape[0], -1)


def unpack(codes):
    q = nibbles(codes)
    return np.where(q >= 8, q - 16, q)


E2M1_MAG = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
E2M1_MID = (E2M1_MAG[1:] + E2M1_MAG[:-1]) / 2          # rounding boundaries of the magnitude


def scale_dev(case_layer, bits):
    """Scales to the device in the precision's dtype (fp16 bits or E4M3 bytes)."""
    return b16(bits, torch.float16) if case_layer["prec"] == 0 else dev(np.asarray(bits, np.uint8))


def scale_values(prec, bits):
    return (oracle.f16_to_f32(bits) if prec == 0 else oracle.e4m3_to_f32(bits)).astype(np.float64)


def run(case, rows=None):
    up, dn = case["up"], case["down"]
    prec = up["prec"]
    codes, scales = oracle.quantize_act(prec, up["x"], up["lam"], alpha=up["alpha_a"])
    xl1 = oracle.lowrank_down(up["x"], up["l1t"]) if up["rank"] else None
    c, s, x = sq.w4a4_gemm_gelu_quant(dev(codes), scale_dev(up, scales), dev(up["w_codes"]),
                                      scale_dev(up, up["w_scales"]), dev(xl1) if up["rank"] else None,
                                      b16(up["l2t"]) if up["rank"] else None, b16(up["bias"]), b16(dn["lam"]),
                                      b16(dn["l1t"]) if dn["rank"] else None, precision=prec,
                                      act_global_scale=up["alpha_a"], w_global_scale=up["alpha_w"],
                                      out_global_scale=dn["alpha_a"])
    # the down projection on the fused outputs; its output width is the
    # up-projection's K, which the GEMM takes only in whole 128-column tiles
    y = None
    if up["K"] % 128 == 0:
        y = sq.w4a4_gemm(prec, c, s, dev(dn["w_codes"]), scale_dev(dn, dn["w_scales"]), x,
                         b16(dn["l2t"]) if dn["rank"] else None, b16(dn["bias"]),
                         act_global_scale=dn["alpha_a"], w_global_scale=dn["alpha_w"])
    torch.cuda.synchronize()
    ref = oracle.mlp_up_gelu_quant(codes, scales, up["w_codes"], up["w_scales"], xl1, up["l2t"], up["bias"],
                                   dn["lam"], dn["l1t"] if dn["rank"] else np.zeros((0, up["N"]), np.uint16),
                                   rows=rows, prec=prec, alpha_a=up["alpha_a"], alpha_w=up["alpha_w"],
                                   alpha_out=dn["alpha_a"])
    ref["up_codes"], ref["up_scales"], ref["up_xl1"] = codes, scales, xl1
    sel = slice(None) if rows is None else np.asarray(rows)
    sc = s.cpu().view(torch.int16).numpy().view(np.uint16) if prec == 0 else s.cpu().numpy()
    full = dict(codes=c.cpu().numpy(), scales=sc, xl1=None if x is None else x.cpu().numpy())
    got = dict(codes=full["codes"][sel], scales=full["scales"][sel],
               xl1=None if x is None else full["xl1"][sel],
               y=None if y is None else y.cpu().view(torch.int16).numpy().view(np.uint16)[sel],
               rows=np.arange(c.shape[0]) if rows is None else np.asarray(rows), full=full)
    return got, ref


C0 = float(np.array([0x3E22F983], np.uint32).view(np.float32)[0])  # the int4 GEMM's accumulator seed
U = 2.0 ** -24  # half an ulp of fp32, relative


def noise_int4(case, rows, ref):
    """Standard deviation of the int4 GEMM's y from its fp32 accumulation: each
    group adds S_g (c0 + P_g 2^-18) to an fp32 accumulator whose magnitude is
    about c0 T_t (T_t = sum of the first t scale products S = sa sw), so its
    rounding is uniform within half an ulp, standard deviation
    2^-24 c0 T_t / sqrt 3, times 2^18 in y; plus the removal of c0 sum S in
    32-group chunks (the matrix instruction's 31 fp32 additions of each chunk
    and one subtraction)."""
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
    return np.sqrt(var)


def noise_nvfp4(case, rows, ref):
    """Standard deviation of the nvfp4 GEMM's y from its fp32 accumulation:
    the products of the dequantized operands are exact, and each 16-channel
    group (one matrix instruction) adds its sum S_g P_g (S = sa sw, P_g the
    group's sum of E2M1 products) to the accumulator, whose value after group
    g is the running sum T_g: one rounding at |T_g| per group, and up to 15
    inside the instruction at about the group's own magnitude, each uniform
    within half an ulp; times alpha_a alpha_w in y."""
    up = case["up"]
    sa = oracle.e4m3_to_f32(ref["up_scales"][rows]).astype(np.float64)       # [R, G]
    sw = oracle.e4m3_to_f32(up["w_scales"]).astype(np.float64)               # [N, G]
    B = sa[:, None, :] * sw[None, :, :] * oracle.group_psums(1, ref["up_codes"][rows], up["w_codes"])
    T = np.cumsum(B, axis=2)
    var = U * U / 3.0 * (np.sum(T * T, axis=2) + 15.0 * np.sum(B * B, axis=2))
    return up["alpha_a"] * up["alpha_w"] * np.sqrt(var)


def flip_model(case, rows, ref):
    """Per h element, the probability that the kernel's bf16(GELU(y)) differs
    from the oracle's bf16(GELU(y)), from an error model of the kernel's y:
      * noise: the fp32 accumulation of the GEMM (noise_int4, noise_nvfp4);
      * a deterministic shift: XL1 rounded to bf16 before the low-rank
        product;
      * a bounded part: fp32 rounding of the global scale, the low-rank
        product, bias and GELU (a few ulp) and the GELU approximation
        (|erf error| < 1.5e-7).
    h is GELU(y) shifted by GELU'(y) times the y error; it flips where the
    shift crosses either end of its bf16 rounding cell."""
    up = case["up"]
    sigma = (noise_int4 if up["prec"] == 0 else noise_nvfp4)(case, rows, ref)
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
    # a bound on the kernel's y error (the shift, 6 sigma of the noise and the
    # bounded part) and the bounded error of its GELU, for the code check
    return dict(p=np.minimum(p, 1.0), y_err=np.abs(shift) + 6.0 * sigma + slack,
                h_err=0.5 * np.abs(y) * 1.5e-7 + 8 * U * np.abs(h))


Y_GELU_MIN = brentq(lambda v: norm.cdf(v) + v * norm.pdf(v), -2.0, -0.1)       # GELU's minimum


def xh_interval(case, ref, model):
    """The range of xh = h / lambda the kernel may have computed: y within
    y_err of the oracle's, GELU over that interval (not monotonic below its
    minimum), its error, the bf16 rounding of h, 1/lambda and the fp32
    rounding of the product."""
    y, ye = ref["y"], model["y_err"]
    ga, gb = oracle.gelu(y - ye)[0], oracle.gelu(y + ye)[0]
    hmin, hmax = np.minimum(ga, gb), np.maximum(ga, gb)
    inside = (y - ye <= Y_GELU_MIN) & (Y_GELU_MIN <= y + ye)
    hmin = np.where(inside, oracle.gelu(np.array([Y_GELU_MIN]))[0][0], hmin)
    hmin, hmax = hmin - model["h_err"], hmax + model["h_err"]
    # the kernel's h is the bf16 rounding to nearest (monotone) of a value in
    # [hmin, hmax]: between the roundings of the ends (taken a little outside,
    # so that the conversion through fp32 cannot move them inward)
    bf = lambda v: synth.bf16_bits_to_f64(oracle.f32_to_bf16(v.astype(np.float32)))
    hmin, hmax = bf(hmin - 2.0 ** -20 * np.abs(hmin)), bf(hmax + 2.0 ** -20 * np.abs(hmax))
    inv_lam = (1.0 / synth.bf16_bits_to_f64(case["down"]["lam"]))[None, :]
    xmin, xmax = hmin * inv_lam, hmax * inv_lam
    return xmin - 2.0 ** -22 * np.abs(xmin), xmax + 2.0 ** -22 * np.abs(xmax)


def t_interval(xmin, xmax, sg):
    """t = xh / (s alpha) for the kernel's own scales sg (s alpha per element),
    with the fp32 roundings of 1/(s alpha) and of the product."""
    d = np.where(sg > 0, sg, 1.0)
    tmin, tmax = xmin / d, xmax / d
    return tmin - 2.0 ** -20 * np.abs(tmin), tmax + 2.0 ** -20 * np.abs(tmax)


def scale_range(prec, xmin, xmax, G, alpha):
    """Per group, the lowest and highest scale the kernel may have written: its
    amax lies between the largest lower bound of |xh| (0 where an interval
    spans 0) and the largest upper bound, and the scale is the precision's
    monotone rounding of amax / 7 (int4, fp16) or amax / (6 alpha) (nvfp4,
    E4M3), each argument within 2^-22 of its fp32 value."""
    R, N = xmin.shape
    lo = np.where((xmin > 0) | (xmax < 0), np.minimum(np.abs(xmin), np.abs(xmax)), 0.0)
    hi = np.maximum(np.abs(xmin), np.abs(xmax))
    alo = lo.reshape(R, N // G, G).max(axis=2)
    ahi = hi.reshape(R, N // G, G).max(axis=2)
    d = 7.0 if prec == 0 else 6.0 * alpha
    alo, ahi = alo / d * (1 - 2.0 ** -22), ahi / d * (1 + 2.0 ** -22)
    if prec == 0:
        return (oracle.f16_to_f32(oracle.f32_to_f16_sat(alo)).astype(np.float64),
                oracle.f16_to_f32(oracle.f32_to_f16_sat(ahi)).astype(np.float64))
    return (oracle.e4m3_to_f32(oracle.f32_to_e4m3_sat(alo)).astype(np.float64),
            oracle.e4m3_to_f32(oracle.f32_to_e4m3_sat(ahi)).astype(np.float64))


def allowance(e):
    return e + 5.0 * np.sqrt(e) + 3.0


def e4m3_near_boundary(bits, arg):
    """Whether arg (the scale's fp32 argument amax / (6 alpha)) lies within 2^-7
    relative of a rounding boundary of the E4M3 code `bits` it rounded to."""
    v = oracle.e4m3_to_f32(bits).astype(np.float64)
    up = oracle.e4m3_to_f32(np.minimum(bits.astype(np.int32) + 1, 0x7E).astype(np.uint8)).astype(np.float64)
    dn = oracle.e4m3_to_f32(np.maximum(bits.astype(np.int32) - 1, 0).astype(np.uint8)).astype(np.float64)
    d = np.minimum(np.abs(arg - (v + up) / 2), np.abs(arg - (v + dn) / 2))
    return d <= 2.0 ** -7 * arg


def e2m1_index(mag, side):
    """Index into E2M1_MAG of the rounding of magnitudes mag to nearest; at a
    tie 'left' gives the lower and 'right' the upper neighbour, so the two
    bound the round-to-nearest-even result whichever neighbour is even."""
    return np.searchsorted(E2M1_MID, mag, side=side)


def check(case, got, ref):
    up, dn = case["up"], case["down"]
    prec = up["prec"]
    G = 64 if prec == 0 else 16
    alpha = 1.0 if prec == 0 else dn["alpha_a"]
    rows = got["rows"]
    s_g, s_o = scale_values(prec, got["scales"]), scale_values(prec, ref["scales"])
    rel = np.abs(s_g - s_o) / np.maximum(s_o, 1e-30)
    xh = ref["xh"].astype(np.float64)
    R, N = xh.shape
    # derived allowances for the number of differing scales and codes
    model = flip_model(case, rows, ref)
    p = model["p"]                                                             # [R, N]
    ax = np.abs(xh).reshape(R, N // G, G)
    near_max = ax >= ax.max(axis=2, keepdims=True) * (1 - 2.0 ** -6)
    ps = np.minimum(1.0, np.sum(p.reshape(R, N // G, G) * near_max, axis=2))   # [R, N/G]
    if prec == 1:
        ps = ps * e4m3_near_boundary(ref["scales"], ax.max(axis=2) / (6.0 * alpha))
    e_s = float(ps.sum())
    # a flip moves xh by at most one bf16 step of h times 1/lambda (and the fp32
    # rounding of the product): the code can change only where a rounding
    # boundary of t = xh / (s alpha) lies that close
    so = np.repeat(s_o, G, axis=1) * alpha
    inv_lam = (1.0 / synth.bf16_bits_to_f64(dn["lam"]))[None, :]
    hstep = np.ldexp(1.0, np.frexp(np.abs(synth.bf16_bits_to_f64(ref["h_bf16"])))[1] - 8)
    t = xh / np.where(so > 0, so, 1.0)
    if prec == 0:
        q_g, q_o = unpack(got["codes"]), unpack(ref["codes"])
        bdist = np.minimum(np.abs(t - (q_o + 0.5)), np.abs(t - (q_o - 0.5)))
    else:
        q_g, q_o = nibbles(got["codes"]), nibbles(ref["codes"])
        bdist = np.min(np.abs(np.abs(t)[..., None] - E2M1_MID), axis=-1)
    reach = so * bdist <= 1.01 * hstep * inv_lam + 2.0 ** -20 * np.abs(xh)
    e_h = float(np.sum(p * reach))
    # codes differ by value: +0 and -0 (E2M1 nibbles 0 and 8) are the same
    diff = q_g != q_o
    if prec == 1:
        diff &= ~(((q_g & 7) == 0) & ((q_o & 7) == 0))
    d_s, d_c = int(np.sum(s_g != s_o)), int(np.sum(diff))
    print(f"[mlp] scales differing {d_s} of {s_g.size} (expected <= {e_s:.1f}, max rel {rel.max():.3g}); "
          f"codes differing {d_c} of {q_g.size} (expected <= {e_h:.1f} from h flips near a code boundary, "
          f"{float(p.sum()):.0f} h flips in all)", flush=True)
    # every scale one the kernel may have written from its own h
    xmin, xmax = xh_interval(case, ref, model)
    smin, smax = scale_range(prec, xmin, xmax, G, alpha)
    bad = (s_g < smin) | (s_g > smax)
    for r_, g_ in np.argwhere(bad)[:6]:
        print(f"[mlp] row {rows[r_]} group {g_}: scale {s_g[r_, g_]:.9g} outside [{smin[r_, g_]:.9g}, "
              f"{smax[r_, g_]:.9g}] (oracle {s_o[r_, g_]:.9g})", flush=True)
    assert not bad.any(), f"{int(bad.sum())} scales outside the range the error model allows"
    assert d_s <= allowance(e_s), f"{d_s} scales differ; the error model allows {allowance(e_s):.1f}"
    assert d_c <= allowance(e_h) + G * d_s, f"{d_c} codes differ; the error model allows {allowance(e_h) + G * d_s:.1f}"
    # every code a rounding of some t the kernel may have quantized, with its own scale
    sg = np.repeat(s_g, G, axis=1) * alpha
    tmin, tmax = t_interval(xmin, xmax, sg)
    if prec == 0:
        ok = (q_g >= np.clip(np.floor(tmin + 0.5), -8, 7)) & (q_g <= np.clip(np.ceil(tmax - 0.5), -8, 7))
        ok |= sg == 0
    else:
        i, neg = q_g & 7, (q_g >> 3) == 1
        # the magnitude range on the code's side of zero (the sign kept at zero)
        mlo = np.where(neg, np.maximum(-tmax, 0.0), np.maximum(tmin, 0.0))
        mhi = np.where(neg, -tmin, tmax)
        ok = np.where(neg, tmin < 0, tmax >= 0)
        ok &= (i >= e2m1_index(mlo, "left")) & (i <= e2m1_index(mhi, "right"))
        ok = np.where(sg > 0, ok, q_g == 0)                                      # a zero scale writes code 0
    if not ok.all():
        for r_, c_ in np.argwhere(~ok)[:12]:
            g_ = c_ // G
            print(f"[mlp] row {rows[r_]} col {c_}: xh {xh[r_, c_]:.9g} t in [{tmin[r_, c_]:.9g}, {tmax[r_, c_]:.9g}] "
                  f"code {q_g[r_, c_]} "
                  f"(oracle {q_o[r_, c_]}), scale {s_g[r_, g_]:.9g} (oracle {s_o[r_, g_]:.9g}), "
                  f"y {ref['y'][r_, c_]:.9g}, h flip p {p[r_, c_]:.3g}", flush=True)
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
    yd, _ = oracle.w4a4_linear(prec, full["codes"], full["scales"], dn["w_codes"], dn["w_scales"],
                               full["xl1"] if dn["rank"] else None, dn["l2t"] if dn["rank"] else None, dn["bias"],
                               alpha_a=dn["alpha_a"], alpha_w=dn["alpha_w"], rows=ri, cols=ci)
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
    # rank_out 48: a second, partly filled 32-rank block of the XL1 products
    "mlp_130x640x256_r48": lambda: synth.mlp_layer(3005, 130, 640, 256, 48),
    "nvfp4_mlp_256x512x256_r16": lambda: synth.mlp_layer(3011, 256, 512, 256, 16, prec=1),
    "nvfp4_mlp_ragged_200x768x384_r32": lambda: synth.mlp_layer(3012, 200, 768, 384, 32, prec=1),
    "nvfp4_mlp_37x256x128_r0": lambda: synth.mlp_layer(3013, 37, 256, 128, 0, prec=1),
    # K = 320, five 64-channel steps; the down projection is not run
    "nvfp4_mlp_ragged_70x384x320_r16": lambda: synth.mlp_layer(3014, 70, 384, 320, 16, prec=1),
    # rank_out 48: a second, partly filled 32-rank block of the XL1 products
    "nvfp4_mlp_130x640x256_r48": lambda: synth.mlp_layer(3015, 130, 640, 256, 48, prec=1),
}


@pytest.mark.parametrize("name", sorted(SMALL))
def test_mlp_fused_small(name):
    print(f"[mlp] {name}", flush=True)
    case = SMALL[name]()
    got, ref = run(case)
    check(case, got, ref)


@pytest.mark.parametrize("prec", [0, 1], ids=["int4", "nvfp4"])
def test_mlp_fused_dit_size_sampled_rows(prec):
    # 1024x1024 diffusion-transformer MLP: 4608 tokens, 3072 -> 12288 -> 3072, rank 32
    print(f"[mlp] dit 4608x12288x3072 prec {prec}", flush=True)
    case = synth.mlp_layer(1002, 4608, 12288, 3072, 32, prec=prec)
    rows = np.concatenate([np.random.default_rng(5).choice(4608, 12, replace=False), [0, 4607]])
    got, ref = run(case, rows=rows)
    check(case, got, ref)
