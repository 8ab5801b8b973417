"""Out-of-bounds write guards: every output of every entry point is placed
inside a larger device buffer whose bytes before and after it hold a poison
pattern, on ragged shapes (M, N or K not a multiple of the kernels' tiles);
after the call the guard bytes must be intact, and the outputs must still
match the oracle (so the whole output was written where it belongs)."""
import numpy as np
import pytest
import torch

import oracle
import bit_w4a4_quantized_smooth_amd as sq
from bit_w4a4_quantized_smooth_amd import synth

pytestmark = pytest.mark.gpu

GUARD = 4096          # bytes of poison on each side
POISON = 0xA5


class Guarded:
    """A device tensor of `shape` / `dtype` with poisoned guard bytes around it."""

    def __init__(self, shape, dtype):
        n = int(np.prod(shape)) * torch.empty((), dtype=dtype).element_size()
        self.n = n
        self.buf = torch.full((GUARD + n + GUARD,), POISON, dtype=torch.uint8, device="cuda")
        self.t = self.buf[GUARD:GUARD + n].view(dtype).view(shape)

    def intact(self):
        b = self.buf.cpu().numpy()
        return bool((b[:GUARD] == POISON).all() and (b[GUARD + self.n:] == POISON).all())


def dev(a, dtype=None):
    if a is None:
        return None
    t = torch.from_numpy(np.ascontiguousarray(a))
    return (t.view(dtype) if dtype is not None else t).cuda()


def b16(bits, dtype=torch.bfloat16):
    return None if bits is None else dev(np.asarray(bits, np.uint16).view(np.int16), dtype)


def host(t):
    t = t.cpu()
    return t.view(torch.int16).numpy().view(np.uint16) if t.dtype in (torch.bfloat16, torch.float16) else t.numpy()


def max_abs_rel(y_bits, ref):
    return float(np.max(np.abs(synth.bf16_bits_to_f64(y_bits) - ref)) / max(np.max(np.abs(ref)), 1e-30))


def sdt(prec):
    return torch.float16 if prec == sq.SVDQ_INT4 else torch.uint8


# quantizer kernels: the first kernel (few rows, rank 0 or 64) and the
# LDS-staged one (ranks 16 / 32 with many rows), ragged rows and channels
QUANT = [(sq.SVDQ_INT4, 37, 320, 16), (sq.SVDQ_INT4, 4130, 2112, 32), (sq.SVDQ_INT4, 45, 576, 0),
         (sq.SVDQ_INT4, 21, 256, 64), (sq.SVDQ_NVFP4, 37, 320, 16), (sq.SVDQ_NVFP4, 4100, 1088, 32)]


# the balanced split of svdq_quantize_act_ws (blocks shared by workgroups):
# ragged last blocks, many-piece blocks, the chunked reciprocal table
QUANT_WS = [(sq.SVDQ_INT4, 1000, 3072, 32), (sq.SVDQ_NVFP4, 2000, 3072, 32), (sq.SVDQ_INT4, 200, 6144, 32),
            (sq.SVDQ_INT4, 3990, 4096, 32)]
_WORK = []


def _work():
    if not _WORK:
        _WORK.append(sq.gemm_workspace())
    return _WORK[0]


@pytest.mark.parametrize("prec,M,K,r,ws", [q + (False,) for q in QUANT] + [q + (True,) for q in QUANT_WS])
def test_quantizer_guards(prec, M, K, r, ws):
    print(f"[guard] quantize prec {prec} {M}x{K} r{r} workspace {ws}", flush=True)
    d = synth.svdq_layer(50 + M, M, 128, K, r, prec, 0.02, 30.0)
    G = sq.GROUP[prec]
    out = (Guarded((M, K // 2), torch.uint8), Guarded((M, K // G), sdt(prec)),
           Guarded((M, r), torch.float32) if r else None)
    sq.quantize_act(prec, b16(d["x"]), b16(d["lam"]), b16(d["l1t"]) if r else None, d["alpha_a"],
                    out=(out[0].t, out[1].t, out[2].t if r else None), workspace=_work() if ws else None)
    torch.cuda.synchronize()
    for g in out:
        assert g is None or g.intact(), "a quantizer output's guard bytes were overwritten"
    oc, os_ = oracle.quantize_act(prec, d["x"], d["lam"], alpha=d["alpha_a"])
    assert np.array_equal(host(out[0].t), oc) and np.array_equal(host(out[1].t), os_)
    if r:
        ox = oracle.lowrank_down(d["x"], d["l1t"])
        assert np.max(np.abs(host(out[2].t) - ox)) <= 1e-4 * np.max(np.abs(ox))


# GEMM grids: small (K-split instance), one-copy with ragged M, nvfp4
GEMM = [(sq.SVDQ_INT4, 200, 256, 1024, 32), (sq.SVDQ_INT4, 2049, 2048, 256, 16), (sq.SVDQ_INT4, 77, 384, 640, 0),
        (sq.SVDQ_NVFP4, 37, 128, 768, 16), (sq.SVDQ_NVFP4, 300, 256, 960, 32)]


def gemm_inputs(prec, M, N, K, r):
    d = synth.svdq_layer(60 + M, M, N, K, r, prec, 0.02, 30.0)
    codes, scales = oracle.quantize_act(prec, d["x"], d["lam"], alpha=d["alpha_a"])
    xl1 = oracle.lowrank_down(d["x"], d["l1t"]) if r else None
    ws = b16(d["w_scales"], torch.float16) if prec == sq.SVDQ_INT4 else dev(d["w_scales"])
    sc = b16(scales, torch.float16) if prec == sq.SVDQ_INT4 else dev(scales)
    return d, codes, scales, xl1, sc, ws


@pytest.mark.parametrize("prec,M,N,K,r", GEMM)
def test_gemm_guards(prec, M, N, K, r):
    print(f"[guard] GEMM prec {prec} {M}x{N}x{K} r{r}", flush=True)
    d, codes, scales, xl1, sc, ws = gemm_inputs(prec, M, N, K, r)
    y = Guarded((M, N), torch.bfloat16)
    sq.w4a4_gemm(prec, dev(codes), sc, dev(d["w_codes"]), ws, dev(xl1), b16(d["l2t"]) if r else None,
                 b16(d["bias"]), d["alpha_a"], d["alpha_w"], out=y.t)
    torch.cuda.synchronize()
    assert y.intact(), "Y's guard bytes were overwritten"
    ref, _ = oracle.w4a4_linear(prec, codes, scales, d["w_codes"], d["w_scales"], xl1, d["l2t"] if r else None,
                                d["bias"], alpha_a=d["alpha_a"], alpha_w=d["alpha_w"])
    assert max_abs_rel(host(y.t), ref) <= 1e-2


@pytest.mark.parametrize("prec,M,N,K", [(sq.SVDQ_INT4, 37, 256, 640), (sq.SVDQ_NVFP4, 45, 128, 320)])
def test_group_psums_guards(prec, M, N, K):
    print(f"[guard] psums prec {prec} {M}x{N}x{K}", flush=True)
    d, codes, *_ = gemm_inputs(prec, M, N, K, 0)
    P = Guarded((M, N, K // sq.GROUP[prec]), torch.int32 if prec == sq.SVDQ_INT4 else torch.float32)
    sq.group_psums(prec, dev(codes), dev(d["w_codes"]), out=P.t)
    torch.cuda.synchronize()
    assert P.intact()
    ref = oracle.group_psums(prec, codes, d["w_codes"])
    assert np.array_equal(P.t.cpu().numpy().view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("prec", [sq.SVDQ_INT4, sq.SVDQ_NVFP4])
def test_qkv_guards(prec):
    print(f"[guard] fused attention projection prec {prec}", flush=True)
    M, H, D, K = 70, 2, 64, 256
    d = synth.qkv_layer(70, M, H, D, K, 16, prec, 0.02, 30.0)
    codes, scales = oracle.quantize_act(prec, d["x"], d["lam"], alpha=d["alpha_a"])
    xl1 = oracle.lowrank_down(d["x"], d["l1t"])
    sc = b16(scales, torch.float16) if prec == sq.SVDQ_INT4 else dev(scales)
    ws = b16(d["w_scales"], torch.float16) if prec == sq.SVDQ_INT4 else dev(d["w_scales"])
    y = Guarded((M, 3 * H * D), torch.bfloat16)
    sq.w4a4_gemm_qkv_norm_rope(prec, dev(codes), sc, dev(d["w_codes"]), ws, dev(xl1), b16(d["l2t"]), b16(d["bias"]),
                               H, D, b16(d["norm_q"]), b16(d["norm_k"]), d["eps"], dev(d["rope"]), d["alpha_a"],
                               d["alpha_w"], out=y.t)
    torch.cuda.synchronize()
    assert y.intact()
    ref, _ = oracle.w4a4_linear_qkv(prec, codes, scales, d["w_codes"], d["w_scales"], xl1, d["l2t"], d["bias"], H, D,
                                    d["norm_q"], d["norm_k"], d["eps"], d["rope"], alpha_a=d["alpha_a"],
                                    alpha_w=d["alpha_w"])
    assert max_abs_rel(host(y.t), ref) <= 1e-2


def test_mlp_guards():
    print("[guard] fused MLP up-projection", flush=True)
    case = synth.mlp_layer(3005, 70, 384, 256, 16)
    up, dn = case["up"], case["down"]
    M, N = 70, 384
    codes, scales = oracle.quantize_act(0, up["x"], up["lam"])
    xl1 = oracle.lowrank_down(up["x"], up["l1t"])
    out = (Guarded((M, N // 2), torch.uint8), Guarded((M, N // 64), torch.float16), Guarded((M, 16), torch.float32))
    sq.w4a4_gemm_gelu_quant(dev(codes), b16(scales, torch.float16), dev(up["w_codes"]),
                            b16(up["w_scales"], torch.float16), dev(xl1), b16(up["l2t"]), b16(up["bias"]),
                            b16(dn["lam"]), b16(dn["l1t"]), out=tuple(g.t for g in out))
    torch.cuda.synchronize()
    for g in out:
        assert g.intact(), "a fused MLP output's guard bytes were overwritten"


@pytest.mark.parametrize("M,N,K", [(2, 320, 1024), (7, 320, 1088), (64, 192, 512)])
def test_awq_guards(M, N, K):
    print(f"[guard] AWQ {M}x{N}x{K}", flush=True)
    d = synth.awq_layer(80 + M, M, N, K)
    y = Guarded((M, N), torch.bfloat16)
    sq.awq_gemv(b16(d["x"]), dev(d["w_codes"]), b16(d["w_scales"], torch.float16), b16(d["w_zeros"], torch.float16),
                b16(d["bias"]), out=y.t)
    torch.cuda.synchronize()
    assert y.intact()
    ref, _ = oracle.awq_linear(d["x"], d["w_codes"], d["w_scales"], d["w_zeros"], d["bias"])
    assert max_abs_rel(host(y.t), ref) <= 1e-2
