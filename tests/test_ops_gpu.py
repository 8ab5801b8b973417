"""The torch custom ops on the GPU: torch.library.opcheck (schema, fake tensor and
AOT-dispatch consistency with the real kernels), a module compiled with
torch.compile(fullgraph=True) against the same module run eagerly (bit-equal:
the same kernels run on the same inputs), and the eager module against the
oracle.
"""
import numpy as np
import pytest
import torch

import oracle
import bit_w4a4_quantized_smooth_amd as sq
from bit_w4a4_quantized_smooth_amd import ops, synth

pytestmark = pytest.mark.gpu


def _t(bits, dtype):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16 if dtype != torch.uint8 else np.uint8)).view(dtype).cuda()


def _svdq_module(d):
    m = ops.SVDQLinear(d["K"], d["N"], rank=d["rank"], precision=d["prec"], bias=d["bias"] is not None, device="cuda")
    sdt = torch.float16 if d["prec"] == sq.SVDQ_INT4 else torch.uint8
    m.smooth.copy_(_t(d["lam"], torch.bfloat16))
    m.w_codes.copy_(_t(d["w_codes"], torch.uint8))
    m.w_scales.copy_(_t(d["w_scales"], sdt))
    if d["rank"]:
        m.l1t.copy_(_t(d["l1t"], torch.bfloat16))
        m.l2t.copy_(_t(d["l2t"], torch.bfloat16))
    if d["bias"] is not None:
        m.bias.copy_(_t(d["bias"], torch.bfloat16))
    m.act_global_scale, m.w_global_scale = d["alpha_a"], d["alpha_w"]
    return m


def _awq_module(d):
    m = ops.AWQLinear(d["K"], d["N"], bias=d["bias"] is not None, device="cuda")
    m.w_codes.copy_(_t(d["w_codes"], torch.uint8))
    m.w_scales.copy_(_t(d["w_scales"], torch.float16))
    m.w_zeros.copy_(_t(d["w_zeros"], torch.float16))
    if d["bias"] is not None:
        m.bias.copy_(_t(d["bias"], torch.bfloat16))
    return m


@pytest.mark.parametrize("prec", [sq.SVDQ_INT4, sq.SVDQ_NVFP4])
def test_opcheck(prec):
    print(f"[ops] opcheck prec {prec}", flush=True)
    d = synth.svdq_layer(31, 96, 256, 512, 16, prec, 0.01, 20.0)
    x = _t(d["x"], torch.bfloat16)
    lam = _t(d["lam"], torch.bfloat16)
    l1t = _t(d["l1t"], torch.bfloat16)
    torch.library.opcheck(torch.ops.svdq.quantize_act.default, (x, lam, l1t, prec, d["alpha_a"]))
    torch.library.opcheck(torch.ops.svdq.quantize_act.default, (x, None, None, prec, d["alpha_a"]))
    codes, scales, xl1 = torch.ops.svdq.quantize_act(x, lam, l1t, prec, d["alpha_a"])
    m = _svdq_module(d)
    torch.library.opcheck(torch.ops.svdq.w4a4_gemm.default,
                          (codes, scales, m.w_codes, m.w_scales, xl1, m.l2t, m.bias, prec, d["alpha_a"], d["alpha_w"]))
    qd = synth.qkv_layer(33, 96, 2, 128, 256, 16, prec)
    qc, qs, qx = torch.ops.svdq.quantize_act(_t(qd["x"], torch.bfloat16), _t(qd["lam"], torch.bfloat16),
                                             _t(qd["l1t"], torch.bfloat16), prec, qd["alpha_a"])
    qm = _svdq_module(qd)
    torch.library.opcheck(torch.ops.svdq.w4a4_gemm_qkv_norm_rope.default,
                          (qc, qs, qm.w_codes, qm.w_scales, qx, qm.l2t, qm.bias, _t(qd["norm_q"], torch.bfloat16),
                           _t(qd["norm_k"], torch.bfloat16), torch.from_numpy(qd["rope"]).cuda(), 2, 128,
                           qd["eps"], prec, qd["alpha_a"], qd["alpha_w"]))
    a = synth.awq_layer(32, 3, 512, 1024)
    am = _awq_module(a)
    torch.library.opcheck(torch.ops.svdq.awq_gemv.default,
                          (_t(a["x"], torch.bfloat16), am.w_codes, am.w_scales, am.w_zeros, am.bias))


@pytest.mark.parametrize("prec", [sq.SVDQ_INT4, sq.SVDQ_NVFP4])
def test_compiled_block_matches_eager(prec):
    print(f"[ops] torch.compile block prec {prec}", flush=True)
    up = synth.svdq_layer(41, 2 * 48, 512, 256, 16, prec, 0.01, 20.0)
    down = synth.svdq_layer(42, 2 * 48, 256, 512, 16, prec, 0.01, 20.0)
    mod = synth.awq_layer(43, 2, 512, 256)
    m_up, m_down, m_mod = _svdq_module(up), _svdq_module(down), _awq_module(mod)
    def block(x, c):
        h = torch.nn.functional.gelu(m_up(x).float()).to(torch.bfloat16) * m_mod(c).unsqueeze(1)
        return m_down(h)

    x = _t(up["x"], torch.bfloat16).reshape(2, 48, 256)
    c = _t(mod["x"], torch.bfloat16)
    y_eager = block(x, c)
    torch._dynamo.reset()
    compiled = torch.compile(block, fullgraph=True, backend="aot_eager")
    for _ in range(2):
        y_comp = compiled(x, c)
        torch.cuda.synchronize()
        assert torch.equal(y_comp.view(torch.int16), y_eager.view(torch.int16))


@pytest.mark.parametrize("prec", [sq.SVDQ_INT4, sq.SVDQ_NVFP4])
def test_module_against_oracle(prec):
    print(f"[ops] SVDQLinear vs oracle prec {prec}", flush=True)
    d = synth.svdq_layer(51, 2 * 40, 384, 512, 32, prec, 0.01, 20.0)
    m = _svdq_module(d)
    y = m(_t(d["x"], torch.bfloat16).reshape(2, 40, 512))
    torch.cuda.synchronize()
    assert y.shape == (2, 40, 384)
    codes, scales = oracle.quantize_act(d["prec"], d["x"], d["lam"], alpha=d["alpha_a"])
    xl1 = oracle.lowrank_down(d["x"], d["l1t"])
    ref, _ = oracle.w4a4_linear(d["prec"], codes, scales, d["w_codes"], d["w_scales"], xl1, d["l2t"], d["bias"],
                                alpha_a=d["alpha_a"], alpha_w=d["alpha_w"])
    got = synth.bf16_bits_to_f64(y.reshape(80, 384).cpu().view(torch.int16).numpy().view(np.uint16))
    assert np.max(np.abs(got - ref)) / np.max(np.abs(ref)) <= 1e-2
