"""Parity of the gfx950 HIP path with the CPU oracle, through the C ABI.

Bar: 4-bit codes, scales and per-group partial products bit-exact; XL1 within
1e-4 of the oracle's double result (normalized by its max |value|); Y within
1e-2 max-abs-rel, max |Y_gpu - y| / max |y| against the oracle's double y
before bf16 rounding.  Small workloads are compared element by element in
full; the DiT-sized ones are compared in full where the oracle is cheap
(codes, scales, XL1, AWQ at M = 2) and on sampled outputs otherwise.
"""
import numpy as np
import pytest
import torch

import oracle
import bit_w4a4_quantized_smooth_amd as sq
from bit_w4a4_quantized_smooth_amd import synth

pytestmark = pytest.mark.gpu

Y_TOL = 1e-2
XL1_TOL = 1e-4


def dev(a, dtype=None):
    if a is None:
        return None
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.view(dtype)
    return t.cuda()


def bf16_dev(bits):
    return dev(np.asarray(bits, np.uint16).view(np.int16), torch.bfloat16)


def f16_dev(bits):
    return dev(np.asarray(bits, np.uint16).view(np.int16), torch.float16)


def host_bits(t):
    t = t.cpu()
    if t.dtype in (torch.bfloat16, torch.float16):
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def bf16_to_f64(bits):
    return synth.bf16_bits_to_f64(bits)


def max_abs_rel(y_bits, y_ref):
    y = bf16_to_f64(y_bits)
    return float(np.max(np.abs(y - y_ref)) / max(np.max(np.abs(y_ref)), 1e-30))


def scales_dev(prec, s):
    return f16_dev(s) if prec == sq.SVDQ_INT4 else dev(s)


def run_quant(d, smooth=True):
    lam = d["lam"] if smooth else None
    codes, scales, xl1 = sq.quantize_act(d["prec"], bf16_dev(d["x"]), bf16_dev(lam) if lam is not None else None,
                                         bf16_dev(d["l1t"]) if d["rank"] else None, d["alpha_a"])
    torch.cuda.synchronize()
    return (host_bits(codes), host_bits(scales), None if xl1 is None else xl1.cpu().numpy())


def check_quant(d, smooth=True):
    codes, scales, xl1 = run_quant(d, smooth)
    lam = d["lam"] if smooth else None
    oc, os_ = oracle.quantize_act(d["prec"], d["x"], lam, alpha=d["alpha_a"])
    assert np.array_equal(scales, os_), f"scales differ at {np.argwhere(scales != os_)[:5]}"
    assert np.array_equal(codes, oc), f"codes differ at {np.argwhere(codes != oc)[:5]}"
    if d["rank"]:
        ox = oracle.lowrank_down(d["x"], d["l1t"])
        err = np.max(np.abs(xl1 - ox)) / max(np.max(np.abs(ox)), 1e-30)
        assert err <= XL1_TOL, err
    return codes, scales, xl1


def run_gemm(d, codes, scales, xl1, with_bias=True):
    y = sq.w4a4_gemm(d["prec"], dev(codes), scales_dev(d["prec"], scales), dev(d["w_codes"]),
                     scales_dev(d["prec"], d["w_scales"]), dev(xl1) if d["rank"] else None,
                     bf16_dev(d["l2t"]) if d["rank"] else None,
                     bf16_dev(d["bias"]) if (with_bias and d["bias"] is not None) else None,
                     d["alpha_a"], d["alpha_w"])
    torch.cuda.synchronize()
    return host_bits(y)


def oracle_y(d, codes, scales, xl1, rows=None, cols=None, with_bias=True):
    y, _ = oracle.w4a4_linear(d["prec"], codes, scales, d["w_codes"], d["w_scales"],
                              xl1 if d["rank"] else None, d["l2t"] if d["rank"] else None,
                              d["bias"] if with_bias else None, alpha_a=d["alpha_a"],
                              alpha_w=d["alpha_w"], rows=rows, cols=cols)
    return y


# --------------------------------------------------------------------------- small, full
SMALL = {
    "int4_256x512x512_r16": lambda: synth.svdq_layer(1001, 256, 512, 512, 16, synth.INT4, 0.01, 20.0),
    "nvfp4_256x512x512_r32": lambda: synth.svdq_layer(1004, 256, 512, 512, 32, synth.NVFP4, 0.01, 20.0),
    "int4_ragged_200x256x1024_r32": lambda: synth.svdq_layer(7, 200, 256, 1024, 32, synth.INT4, 0.02, 30.0),
    "nvfp4_ragged_37x128x768_r16": lambda: synth.svdq_layer(8, 37, 128, 768, 16, synth.NVFP4, 0.02, 30.0),
    "int4_rank0_130x384x320": lambda: synth.svdq_layer(9, 130, 384, 320, 0, synth.INT4, 0.01, 20.0),
    "int4_rank128_64x128x256": lambda: synth.svdq_layer(10, 64, 128, 256, 128, synth.INT4, 0.01, 20.0),
    # int4 with an even group count and 1, 5, 7 two-group stages: the GEMM
    # loads scales in blocks of four stages
    "int4_k64_50x128x64_r16": lambda: synth.svdq_layer(19, 50, 128, 64, 16, synth.INT4, 0.02, 30.0),
    "int4_k128_40x128x128_r16": lambda: synth.svdq_layer(15, 40, 128, 128, 16, synth.INT4, 0.02, 30.0),
    "int4_k640_ragged_77x256x640_r32": lambda: synth.svdq_layer(16, 77, 256, 640, 32, synth.INT4, 0.02, 30.0),
    "int4_k896_rank0_130x128x896": lambda: synth.svdq_layer(17, 130, 128, 896, 0, synth.INT4, 0.01, 20.0),
    # NVFP4 K steps of 64 channels not a multiple of four (1, 5, 6, 7): the
    # GEMM stages codes two steps and scales sixteen steps at a time
    "nvfp4_k64_33x128x64_r16": lambda: synth.svdq_layer(11, 33, 128, 64, 16, synth.NVFP4, 0.02, 30.0),
    "nvfp4_k320_ragged_45x256x320_r16": lambda: synth.svdq_layer(12, 45, 256, 320, 16, synth.NVFP4, 0.02, 30.0),
    "nvfp4_k384_96x384x384_r32": lambda: synth.svdq_layer(13, 96, 384, 384, 32, synth.NVFP4, 0.01, 20.0),
    "nvfp4_k448_rank0_70x128x448": lambda: synth.svdq_layer(14, 70, 128, 448, 0, synth.NVFP4, 0.01, 20.0),
    # and 15 (a whole remainder) and 17 (one 16-step scale block and one more)
    "nvfp4_k960_ragged_33x256x960_r16": lambda: synth.svdq_layer(20, 33, 256, 960, 16, synth.NVFP4, 0.02, 30.0),
    "nvfp4_k1088_64x128x1088_r32": lambda: synth.svdq_layer(21, 64, 128, 1088, 32, synth.NVFP4, 0.01, 20.0),
}


@pytest.fixture(scope="module", params=sorted(SMALL))
def small(request):
    print(f"[parity] case {request.param}", flush=True)
    return SMALL[request.param]()


def test_quantize_small(small):
    check_quant(small)


def test_quantize_without_smoothing(small):
    check_quant(small, smooth=False)


def test_group_psums_small(small):
    d = small
    codes, _ = oracle.quantize_act(d["prec"], d["x"], d["lam"], alpha=d["alpha_a"])
    P = sq.group_psums(d["prec"], dev(codes), dev(d["w_codes"]))
    torch.cuda.synchronize()
    ref = oracle.group_psums(d["prec"], codes, d["w_codes"])
    got = P.cpu().numpy()
    assert got.dtype == ref.dtype
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


def test_gemm_small(small):
    d = small
    codes, scales = oracle.quantize_act(d["prec"], d["x"], d["lam"], alpha=d["alpha_a"])
    xl1 = oracle.lowrank_down(d["x"], d["l1t"]) if d["rank"] else None
    y = run_gemm(d, codes, scales, xl1)
    ref = oracle_y(d, codes, scales, xl1)
    assert max_abs_rel(y, ref) <= Y_TOL
    yn = run_gemm(d, codes, scales, xl1, with_bias=False)
    refn = oracle_y(d, codes, scales, xl1, with_bias=False)
    assert max_abs_rel(yn, refn) <= Y_TOL


def test_linear_end_to_end_small(small):
    d = small
    codes, scales, xl1 = check_quant(d)
    y = run_gemm(d, codes, scales, xl1)
    oc, os_ = oracle.quantize_act(d["prec"], d["x"], d["lam"], alpha=d["alpha_a"])
    ox = oracle.lowrank_down(d["x"], d["l1t"]) if d["rank"] else None
    ref = oracle_y(d, oc, os_, ox)
    assert max_abs_rel(y, ref) <= Y_TOL


# --------------------------------------------------------------------------- largest K
# The quantizer's largest K (32768): 16 chunks of 2048 channels in the
# LDS-staged kernel (int4, 4112 rows), 512 steps in the first kernel (nvfp4,
# 40 rows).  The GEMM over 512 groups: its fp32 accumulator carries
# c0 * sum_g S for all of them until the epilogue removes it.
@pytest.mark.parametrize("prec,M,rank", [(sq.SVDQ_INT4, 4112, 32), (sq.SVDQ_NVFP4, 40, 16)])
def test_quantize_max_k(prec, M, rank):
    print(f"[parity] quantize {M}x32768 prec {prec} r{rank}", flush=True)
    check_quant(synth.svdq_layer(40 + prec, M, 128, 32768, rank, prec, 0.005, 30.0))


@pytest.mark.parametrize("prec", [sq.SVDQ_INT4, sq.SVDQ_NVFP4])
def test_gemm_max_k(prec):
    print(f"[parity] GEMM 64x256x32768 prec {prec}", flush=True)
    d = synth.svdq_layer(42 + prec, 64, 256, 32768, 16, prec, 0.01, 20.0)
    codes, scales = oracle.quantize_act(d["prec"], d["x"], d["lam"], alpha=d["alpha_a"])
    xl1 = oracle.lowrank_down(d["x"], d["l1t"])
    y = run_gemm(d, codes, scales, xl1)
    err = max_abs_rel(y, oracle_y(d, codes, scales, xl1))
    print(f"[parity] max-abs-rel {err:.2e}", flush=True)
    assert err <= Y_TOL


# --------------------------------------------------------------------------- int4 GEMM grid sizes
# A grid of at most one 128x128 tile per CU (256 on MI355X) with K % 256 == 0
# runs on the K-split kernel (two copies of the workgroup, each half of K);
# one more tile row goes back to the plain grid.  Sampled rows (first, last,
# and spread) and all columns against the oracle.
@pytest.mark.parametrize("M", [2048, 2049])
def test_gemm_split_boundary(M):
    print(f"[parity] int4 GEMM {M}x2048x256 (tiles {((M + 127) // 128) * 16})", flush=True)
    d = synth.svdq_layer(18, M, 2048, 256, 16, synth.INT4, 0.01, 20.0)
    codes, scales = oracle.quantize_act(d["prec"], d["x"], d["lam"], alpha=d["alpha_a"])
    xl1 = oracle.lowrank_down(d["x"], d["l1t"])
    y = run_gemm(d, codes, scales, xl1)
    rr, cc = np.meshgrid(np.unique(np.concatenate([np.arange(0, M, 61), [M - 1]])), np.arange(2048), indexing="ij")
    ref = oracle_y(d, codes, scales, xl1, rows=rr.ravel(), cols=cc.ravel())
    assert max_abs_rel(y[rr.ravel(), cc.ravel()], ref) <= Y_TOL


# --------------------------------------------------------------------------- quantizer, many rows
# int4 with ranks 16 / 32 on more 16-row blocks than the device has CUs goes to
# the LDS-staged quantizer (32 rows per workgroup, one ring over all of K with
# lambda reciprocals in 2048-channel chunks): the DiT attention input, ragged
# rows and channels (a partial last workgroup, a partial last chunk, a
# one-step chunk), a single 64-channel step, and no smoothing factor.
MANY_ROWS = {
    "int4_4608x3072_r32": lambda: synth.svdq_layer(1002, 4608, 128, 3072, 32, synth.INT4, 0.005, 30.0),
    "int4_ragged_4100x4160_r16": lambda: synth.svdq_layer(31, 4100, 128, 4160, 16, synth.INT4, 0.02, 30.0),
    "int4_ragged_4130x2112_r32": lambda: synth.svdq_layer(32, 4130, 128, 2112, 32, synth.INT4, 0.02, 30.0),
    "int4_4200x64_r32": lambda: synth.svdq_layer(33, 4200, 128, 64, 32, synth.INT4, 0.02, 30.0),
    "nvfp4_4608x3072_r32": lambda: synth.svdq_layer(1004, 4608, 128, 3072, 32, synth.NVFP4, 0.005, 30.0),
    # no smoothing factor (lambda = 1), and nvfp4 on ragged rows with a one-step last chunk
    "int4_nosmooth_4112x2176_r16": lambda: synth.svdq_layer(34, 4112, 128, 2176, 16, synth.INT4, 0.02, 30.0,
                                                             smooth=False),
    "nvfp4_ragged_4100x4160_r16": lambda: synth.svdq_layer(35, 4100, 128, 4160, 16, synth.NVFP4, 0.02, 30.0),
}


@pytest.mark.parametrize("name", sorted(MANY_ROWS))
def test_quantize_many_rows(name):
    print(f"[parity] quantize {name}", flush=True)
    check_quant(MANY_ROWS[name]())


# --------------------------------------------------------------------------- quantizer edge cases
def _bits(a):
    return synth.to_bf16_bits(np.asarray(a, np.float64))


def _edge_case(prec, kind):
    G = 64 if prec == sq.SVDQ_INT4 else 16
    M, K = 48, 256
    rng = np.random.default_rng(11)
    if kind == "ties":
        # x = (q + 1/2) * s with s a power of two: exact midpoints of the code grid
        s = 2.0 ** rng.integers(-8, 4, size=(M, K // G))
        q = rng.integers(-7, 7, size=(M, K)) + 0.5
        x = q * np.repeat(s, G, axis=1)
        x[:, ::G] = 7.0 * np.repeat(s, G, axis=1)[:, ::G]
    elif kind == "tiny":
        x = rng.standard_normal((M, K)) * 1e-6  # fp16-subnormal / E4M3-underflow scales
    elif kind == "huge":
        x = rng.standard_normal((M, K)) * 3e5  # fp16 scale saturates at 65504
    elif kind == "zeros":
        x = np.zeros((M, K))
        x[1::2, :G] = rng.standard_normal((M // 2, G))
    elif kind == "grid":
        # E2M1 values and the midpoints between them, both signs, and signed
        # zeros, times a power-of-two scale s per group whose first entry is
        # 6 s: with alpha = 1 the NVFP4 scale is s exactly and x / s is exact,
        # so every code decision is a tie or an exact grid point.  Rows 0 mod 5
        # hold groups of -0 only (scale 0: code 0, not the negative zero).
        mags = np.array([0.0, 0.25, 0.5, 0.75, 1.0, 1.25, 1.5, 1.75, 2.0, 2.5, 3.0, 3.5, 4.0, 5.0, 6.0])
        s = 2.0 ** rng.integers(-6, 8, size=(M, K // G))
        x = rng.choice(mags, size=(M, K)) * np.where(rng.random((M, K)) < 0.5, -1.0, 1.0)
        x[:, ::G] = 6.0 * np.where(rng.random((M, K // G)) < 0.5, -1.0, 1.0)
        x = x * np.repeat(s, G, axis=1)
        x[::5, :] = -0.0
    elif kind == "inf":
        x = rng.standard_normal((M, K))
        x[rng.random((M, K)) < 0.01] = np.inf
        x[rng.random((M, K)) < 0.01] = -np.inf
    fixed_alpha = prec == sq.SVDQ_INT4 or kind in ("grid", "inf")
    return dict(prec=prec, x=_bits(x), lam=None, rank=0, alpha_a=1.0 if fixed_alpha else
                synth.nvfp4_act_global_scale(_bits(x), None), l1t=np.zeros((0, K), np.uint16))


@pytest.mark.parametrize("prec", [sq.SVDQ_INT4, sq.SVDQ_NVFP4])
@pytest.mark.parametrize("kind", ["ties", "tiny", "huge", "zeros", "grid", "inf"])
def test_quantize_edge_cases(prec, kind):
    print(f"[parity] quantize edge {kind} prec {prec}", flush=True)
    check_quant(_edge_case(prec, kind), smooth=False)


@pytest.mark.parametrize("prec", [sq.SVDQ_INT4, sq.SVDQ_NVFP4])
def test_empty_inputs(prec):
    d = synth.svdq_layer(1, 0, 128, 256, 16, prec)
    codes, scales, xl1 = sq.quantize_act(prec, bf16_dev(np.zeros((0, 256), np.uint16)), None,
                                         bf16_dev(d["l1t"]), 1.0 if prec == sq.SVDQ_INT4 else 0.01)
    y = sq.w4a4_gemm(prec, codes, scales, dev(d["w_codes"]), scales_dev(prec, d["w_scales"]), xl1,
                     bf16_dev(d["l2t"]), None, d["alpha_a"], d["alpha_w"])
    torch.cuda.synchronize()
    assert codes.shape == (0, 128) and xl1.shape == (0, 16) and y.shape == (0, 128)


def test_awq_empty_input():
    a = synth.awq_layer(2, 1, 256, 512)
    y = sq.awq_gemv(bf16_dev(np.zeros((0, 512), np.uint16)), dev(a["w_codes"]), f16_dev(a["w_scales"]),
                    f16_dev(a["w_zeros"]), bf16_dev(a["bias"]))
    torch.cuda.synchronize()
    assert y.shape == (0, 256)


# --------------------------------------------------------------------------- AWQ
AWQ = {
    "awq_2x18432x3072": lambda: synth.awq_layer(1005, 2, 18432, 3072),
    "awq_1x512x512": lambda: synth.awq_layer(21, 1, 512, 512),
    "awq_5x1024x1024_nobias": lambda: synth.awq_layer(22, 5, 1024, 1024, with_bias=False),
    "awq_64x1024x3072": lambda: synth.awq_layer(23, 64, 1024, 3072),
    "awq_2x256x5120": lambda: synth.awq_layer(24, 2, 256, 5120),
    "awq_3x8192x1024": lambda: synth.awq_layer(25, 3, 8192, 1024),
    "awq_2x3072x8192": lambda: synth.awq_layer(26, 2, 3072, 8192),
    "awq_4x192x1536": lambda: synth.awq_layer(27, 4, 192, 1536, with_bias=False),
    # K not a multiple of 512 (the LDS-staged matrix-core kernel): an odd
    # group count (a last stage of one group), an odd number of two-group
    # stages, and many 64-row workgroups
    "awq_7x320x1088": lambda: synth.awq_layer(28, 7, 320, 1088),
    "awq_64x256x192": lambda: synth.awq_layer(29, 64, 256, 192),
    "awq_8x24576x256": lambda: synth.awq_layer(30, 8, 24576, 256),
    # streamed kernel: 34 chunks of K (more than the ring holds) on 8 CUs
    "awq_6x128x17408": lambda: synth.awq_layer(31, 6, 128, 17408),
    "awq_33x4096x3072_nobias": lambda: synth.awq_layer(32, 33, 4096, 3072, with_bias=False),
    # the streamed kernel's batch shapes on 256 CUs: 4 units per workgroup,
    # 5 + 3 (two batches), 5 units at two m-blocks, 2 at three, 2-3 (ragged)
    "awq_16x16384x1024": lambda: synth.awq_layer(33, 16, 16384, 1024),
    "awq_8x32768x512": lambda: synth.awq_layer(34, 8, 32768, 512),
    "awq_24x20480x512": lambda: synth.awq_layer(35, 24, 20480, 512),
    "awq_48x8192x2048": lambda: synth.awq_layer(36, 48, 8192, 2048),
    "awq_12x9216x1536": lambda: synth.awq_layer(37, 12, 9216, 1536),
}


@pytest.mark.parametrize("name", sorted(AWQ))
def test_awq(name):
    print(f"[parity] {name}", flush=True)
    d = AWQ[name]()
    y = sq.awq_gemv(bf16_dev(d["x"]), dev(d["w_codes"]), f16_dev(d["w_scales"]), f16_dev(d["w_zeros"]),
                    bf16_dev(d["bias"]) if d["bias"] is not None else None)
    torch.cuda.synchronize()
    ref, _ = oracle.awq_linear(d["x"], d["w_codes"], d["w_scales"], d["w_zeros"], d["bias"])
    assert max_abs_rel(host_bits(y), ref) <= Y_TOL


def test_awq_modulation_m64_sampled():
    d = synth.awq_layer(1005, 64, 18432, 3072)
    y = sq.awq_gemv(bf16_dev(d["x"]), dev(d["w_codes"]), f16_dev(d["w_scales"]), f16_dev(d["w_zeros"]),
                    bf16_dev(d["bias"]))
    torch.cuda.synchronize()
    rng = np.random.default_rng(3)
    rows = rng.integers(0, 64, 4096)
    cols = rng.integers(0, 18432, 4096)
    ref, _ = oracle.awq_linear(d["x"], d["w_codes"], d["w_scales"], d["w_zeros"], d["bias"], rows=rows, cols=cols)
    yb = host_bits(y)[rows, cols]
    assert max_abs_rel(yb, ref) <= Y_TOL
