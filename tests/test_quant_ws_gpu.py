"""The balanced quantizer (svdq_quantize_act_ws) against the CPU oracle and
against svdq_quantize_act, through the C ABI.

The call's (32-row block, 64-channel step) grid is cut into equal ranges, one
per workgroup, so a block can be shared by several workgroups whose XL1 pieces
meet in the workspace.  Codes and scales are the same function of the inputs
as in the plain call (bit-exact, also against the oracle: formats from
"Nunchaku Lite", "Supported quantization types"); XL1 (blog "Nunchaku 4-bit
inference in Diffusers", "Background: SVDQuant and Nunchaku": the fused
down-projection) within 1e-4 of the oracle's double result, normalized by its
largest magnitude, and bit-identical from call to call.  Shapes cover blocks
split in two and in many pieces, a ragged last block, the chunked reciprocal
table (K > 4096), the fallbacks to the plain kernel, and back-to-back calls of
different shapes on one workspace (the counters must come back to zero).
"""
import numpy as np
import pytest
import torch

import oracle
import bit_w4a4_quantized_smooth_amd as sq
from bit_w4a4_quantized_smooth_amd import synth

pytestmark = pytest.mark.gpu

XL1_TOL = 1e-4

# (precision, M, K, rank): split with two-piece blocks (3990 x 4096 with a
# ragged last block; the MLP-down input 4608 x 12288 with the chunked
# reciprocal table), many-piece blocks (1000 x 3072, 2000 x 3072 nvfp4 and
# rank 16, 200 x 6144 chunked), and the cases where the split does not apply
# and the call is the plain one (the QKV input 4608 x 3072: it would save
# fewer than eight rounds; K = 4608: 72 steps are not whole 2048-channel
# chunks; M = 8192: as many blocks as CUs; tiny calls)
CASES = [(sq.SVDQ_INT4, 3990, 4096, 32), (sq.SVDQ_INT4, 4608, 12288, 32), (sq.SVDQ_INT4, 1000, 3072, 32),
         (sq.SVDQ_NVFP4, 2000, 3072, 32), (sq.SVDQ_INT4, 2000, 3072, 16), (sq.SVDQ_INT4, 200, 6144, 32),
         (sq.SVDQ_INT4, 4608, 3072, 32), (sq.SVDQ_NVFP4, 4608, 3072, 32), (sq.SVDQ_INT4, 70, 4608, 32),
         (sq.SVDQ_INT4, 8192, 1024, 16), (sq.SVDQ_NVFP4, 33, 1024, 16), (sq.SVDQ_INT4, 1, 256, 16)]


def b16(bits, dtype=torch.bfloat16):
    if bits is None:
        return None
    return torch.from_numpy(np.ascontiguousarray(np.asarray(bits, np.uint16).view(np.int16))).view(dtype).cuda()


def host(t):
    t = t.cpu()
    return t.view(torch.int16).numpy().view(np.uint16) if t.dtype in (torch.bfloat16, torch.float16) else t.numpy()


@pytest.fixture(scope="module")
def work():
    return sq.gemm_workspace()


@pytest.mark.parametrize("prec,M,K,r", CASES)
def test_balanced_quantizer(prec, M, K, r, work):
    print(f"[quant_ws] prec {prec} {M}x{K} r{r}", flush=True)
    d = synth.svdq_layer(700 + M % 97, M, 128, K, r, prec, 0.02, 30.0)
    x, lam, l1t = b16(d["x"]), b16(d["lam"]), b16(d["l1t"])
    c1, s1, x1 = sq.quantize_act(prec, x, lam, l1t, d["alpha_a"], workspace=work)
    c2, s2, x2 = sq.quantize_act(prec, x, lam, l1t, d["alpha_a"], workspace=work)
    c0, s0, x0 = sq.quantize_act(prec, x, lam, l1t, d["alpha_a"])
    torch.cuda.synchronize()
    codes, scales, xl1 = host(c1), host(s1), host(x1)
    assert np.array_equal(codes, host(c0)) and np.array_equal(scales, host(s0)), "codes / scales differ from the plain call"
    assert np.array_equal(xl1.view(np.uint32), host(x2).view(np.uint32)), "XL1 differs between two calls"
    oc, os_ = oracle.quantize_act(prec, d["x"], d["lam"], alpha=d["alpha_a"])
    assert np.array_equal(scales, os_), f"scales differ at {np.argwhere(scales != os_)[:5]}"
    assert np.array_equal(codes, oc), f"codes differ at {np.argwhere(codes != oc)[:5]}"
    ox = oracle.lowrank_down(d["x"], d["l1t"])
    err = float(np.max(np.abs(xl1 - ox)) / max(np.max(np.abs(ox)), 1e-30))
    err0 = float(np.max(np.abs(host(x0) - ox)) / max(np.max(np.abs(ox)), 1e-30))
    print(f"[quant_ws] XL1 max-abs-rel {err:.2e} (plain call {err0:.2e})", flush=True)
    assert err <= XL1_TOL, err
    # the workspace's quantizer counters are zero again after the calls
    cnt = work[sq.GEMM_WORK_BYTES - 4096 + 1024:sq.GEMM_WORK_BYTES - 4096 + 3072].cpu().numpy()
    assert not cnt.any(), "quantizer counters left non-zero"


def test_rank0_and_empty_with_workspace(work):
    d = synth.svdq_layer(711, 300, 128, 512, 0, sq.SVDQ_INT4, 0.02, 30.0)
    c, s, xl1 = sq.quantize_act(sq.SVDQ_INT4, b16(d["x"]), b16(d["lam"]), None, workspace=work)
    torch.cuda.synchronize()
    assert xl1 is None
    oc, os_ = oracle.quantize_act(sq.SVDQ_INT4, d["x"], d["lam"])
    assert np.array_equal(host(c), oc) and np.array_equal(host(s), os_)
    e = torch.empty((0, 512), dtype=torch.bfloat16, device="cuda")
    c, s, xl1 = sq.quantize_act(sq.SVDQ_INT4, e, None, torch.zeros((16, 512), dtype=torch.bfloat16, device="cuda"),
                                workspace=work)
    assert c.shape == (0, 256) and xl1.shape == (0, 16)
