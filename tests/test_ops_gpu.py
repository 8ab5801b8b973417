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
    torch.library.opcheck(torch.ops.svdq.w4a4_gemm_ws.default,
                          (codes, scales, m.w_codes, m.w_scales, xl1, m.l2t, m.bias, sq.gemm_workspace(), prec,
                           d["alpha_a"], d["alpha_w"]))
    # the balanced quantizer splits this one (1000 rows, 48 steps of a block, rank 32)
    ds = synth.svdq_layer(34, 1000, 128, 3072, 32, prec, 0.01, 20.0)
    torch.library.opcheck(torch.ops.svdq.quantize_act_ws.default,
                          (_t(ds["x"], torch.bfloat16), _t(ds["lam"], torch.bfloat16), _t(ds["l1t"], torch.bfloat16),
                           sq.gemm_workspace(), prec, ds["alpha_a"]))
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


def _mlp_module(case):
    up, dn = case["up"], case["down"]
    prec = up["prec"]
    m = ops.SVDQMLP(up["K"], up["N"], rank=up["rank"], precision=prec, device="cuda")
    sdt = torch.float16 if prec == sq.SVDQ_INT4 else torch.uint8
    for lin, d in ((m.up, up), (m.down, dn)):
        if "lam" in d:
            lin.smooth.copy_(_t(d["lam"], torch.bfloat16))
        lin.w_codes.copy_(_t(d["w_codes"], torch.uint8))
        lin.w_scales.copy_(_t(d["w_scales"], sdt))
        lin.l1t.copy_(_t(d["l1t"], torch.bfloat16))
        lin.l2t.copy_(_t(d["l2t"], torch.bfloat16))
        lin.bias.copy_(_t(d["bias"], torch.bfloat16))
        lin.act_global_scale, lin.w_global_scale = float(d["alpha_a"]), float(d["alpha_w"])
    return m


@pytest.mark.parametrize("prec", [sq.SVDQ_INT4, sq.SVDQ_NVFP4])
def test_mlp_op_and_module(prec):
    # 96 tokens, 256 -> 512 -> 256, rank 16: opcheck of the fused operator,
    # the compiled module bit-equal to eager, and the module's output against the
    # oracle's down projection of the fused kernel's own codes, scales and XL1
    # (the fused quantization itself is compared in tests/test_mlp_gpu.py)
    print(f"[ops] SVDQMLP precision {prec}", flush=True)
    case = synth.mlp_layer(61, 96, 512, 256, 16, prec)
    up, dn = case["up"], case["down"]
    m = _mlp_module(case)
    x = _t(up["x"], torch.bfloat16)
    ga = (m.up.act_global_scale, m.up.w_global_scale, m.down.act_global_scale)
    codes, scales, xl1 = torch.ops.svdq.quantize_act(x, m.up.smooth, m.up.l1t, prec, ga[0])
    torch.library.opcheck(torch.ops.svdq.w4a4_gemm_gelu_quant.default,
                          (codes, scales, m.up.w_codes, m.up.w_scales, xl1, m.up.l2t, m.up.bias, m.down.smooth,
                           m.down.l1t, prec, *ga))
    y_eager = m(x.reshape(2, 48, 256))
    torch._dynamo.reset()
    compiled = torch.compile(m, fullgraph=True, backend="aot_eager")
    for _ in range(2):
        y_comp = compiled(x.reshape(2, 48, 256))
        torch.cuda.synchronize()
        assert torch.equal(y_comp.view(torch.int16), y_eager.view(torch.int16))
    hc, hs, hx = torch.ops.svdq.w4a4_gemm_gelu_quant(codes, scales, m.up.w_codes, m.up.w_scales, xl1, m.up.l2t,
                                                     m.up.bias, m.down.smooth, m.down.l1t, prec, *ga)
    torch.cuda.synchronize()
    hs_np = hs.cpu().view(torch.int16).numpy().view(np.uint16) if prec == sq.SVDQ_INT4 else hs.cpu().numpy()
    ref, _ = oracle.w4a4_linear(prec, hc.cpu().numpy(), hs_np, dn["w_codes"], dn["w_scales"], hx.cpu().numpy(),
                                dn["l2t"], dn["bias"], alpha_a=dn["alpha_a"], alpha_w=dn["alpha_w"])
    got = synth.bf16_bits_to_f64(y_eager.reshape(96, 256).cpu().view(torch.int16).numpy().view(np.uint16))
    e = np.max(np.abs(got - ref)) / np.max(np.abs(ref))
    print(f"[ops] SVDQMLP vs oracle on the fused outputs: max-abs-rel {e:.2e}", flush=True)
    assert e <= 1e-2


@pytest.mark.parametrize("prec", [sq.SVDQ_INT4, sq.SVDQ_NVFP4])
def test_module_with_workspace(prec):
    # the QKV projection's size (4608 tokens, 3072 -> 9216, rank 32), where the
    # GEMM grid's last round is split: the layer with a workspace against the
    # same layer without (every output outside the 32 split tiles equal, the
    # rest within the int4 conversion noise), and compiled against eager bit
    # for bit, the workspace's counter words left zero
    print(f"[ops] SVDQLinear with a workspace, prec {prec}", flush=True)
    d = synth.svdq_layer(71, 4608, 9216, 3072, 32, prec, 0.005, 30.0)
    m = _svdq_module(d)
    x = _t(d["x"], torch.bfloat16).reshape(2, 2304, 3072)
    y_plain = m(x)
    m.workspace = ops.gemm_workspace()
    y_ws = m(x)
    torch.cuda.synchronize()
    assert int(m.workspace[:16 << 20].count_nonzero()) > 0, "no partial tile written: no split ran"
    assert int(m.workspace[16 << 20:].count_nonzero()) == 0
    n_diff = int((y_ws.view(torch.int16) != y_plain.view(torch.int16)).sum())
    assert n_diff <= 32 * 128 * 128
    rel = float((y_ws.float() - y_plain.float()).abs().max() / y_plain.float().abs().max())
    print(f"[ops] {n_diff} outputs differ from the layer without a workspace, max-abs-rel {rel:.1e}", flush=True)
    assert rel <= 1e-2
    torch._dynamo.reset()
    compiled = torch.compile(m, fullgraph=True, backend="aot_eager")
    for _ in range(2):
        y_comp = compiled(x)
        torch.cuda.synchronize()
        assert torch.equal(y_comp.view(torch.int16), y_ws.view(torch.int16))
    assert int(m.workspace[16 << 20:].count_nonzero()) == 0


@pytest.mark.parametrize("prec", [sq.SVDQ_INT4, sq.SVDQ_NVFP4])
def test_module_with_workspace_split_quantizer(prec):
    # 1000 tokens (31 full 32-row blocks and a ragged one, fewer than the CUs):
    # the quantizer splits each block over several workgroups.  Against the
    # same layer without a workspace: codes and scales are the same, XL1 of
    # the shared blocks differs in its last bits, so Y stays within the int4
    # conversion noise; compiled equals eager bit for bit; counters zero.
    print(f"[ops] SVDQLinear 1000 tokens with a workspace, prec {prec}", flush=True)
    d = synth.svdq_layer(72, 1000, 1024, 3072, 32, prec, 0.005, 30.0)
    m = _svdq_module(d)
    x = _t(d["x"], torch.bfloat16)
    y_plain = m(x)
    m.workspace = ops.gemm_workspace()
    y_ws = m(x)
    torch.cuda.synchronize()
    assert int(m.workspace[:16 << 20].count_nonzero()) > 0, "no partial tile written: no split ran"
    assert int(m.workspace[16 << 20:].count_nonzero()) == 0
    rel = float((y_ws.float() - y_plain.float()).abs().max() / y_plain.float().abs().max())
    print(f"[ops] max-abs-rel against the layer without a workspace {rel:.1e}", flush=True)
    assert rel <= 1e-2
    torch._dynamo.reset()
    compiled = torch.compile(m, fullgraph=True, backend="aot_eager")
    for _ in range(2):
        y_comp = compiled(x)
        torch.cuda.synchronize()
        assert torch.equal(y_comp.view(torch.int16), y_ws.view(torch.int16))
    assert int(m.workspace[16 << 20:].count_nonzero()) == 0
