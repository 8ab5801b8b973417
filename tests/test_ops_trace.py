"""The torch custom-op layer (svdq::quantize_act, svdq::w4a4_gemm,
svdq::w4a4_gemm_qkv_norm_rope, svdq::w4a4_gemm_gelu_quant, svdq::awq_gemv):
fake implementations give the shapes and dtypes the C ABI documents, and a
module built on them traces as one graph (torch.export in strict mode goes
through the same frontend as torch.compile(fullgraph=True)).  Tracing uses
fake tensors only, so no kernel runs and this file needs no GPU.
"""
import pytest
import torch
from torch._subclasses.fake_tensor import FakeTensorMode

import bit_w4a4_quantized_smooth_amd as sq
from bit_w4a4_quantized_smooth_amd import ops


@pytest.mark.parametrize("prec", [sq.SVDQ_INT4, sq.SVDQ_NVFP4])
@pytest.mark.parametrize("rank", [0, 32])
def test_fake_shapes(prec, rank):
    M, K, N = 96, 512, 384
    G = sq.GROUP[prec]
    sdt = torch.float16 if prec == sq.SVDQ_INT4 else torch.uint8
    with FakeTensorMode():
        x = torch.empty(M, K, dtype=torch.bfloat16)
        lam = torch.empty(K, dtype=torch.bfloat16)
        l1t = torch.empty(rank, K, dtype=torch.bfloat16) if rank else None
        codes, scales, xl1 = torch.ops.svdq.quantize_act(x, lam, l1t, prec, 1.0)
        assert (codes.shape, codes.dtype) == ((M, K // 2), torch.uint8)
        assert (scales.shape, scales.dtype) == ((M, K // G), sdt)
        assert (xl1.shape, xl1.dtype) == ((M, rank), torch.float32)
        wc = torch.empty(N, K // 2, dtype=torch.uint8)
        ws = torch.empty(N, K // G, dtype=sdt)
        l2t = torch.empty(N, rank, dtype=torch.bfloat16) if rank else None
        y = torch.ops.svdq.w4a4_gemm(codes, scales, wc, ws, xl1, l2t, None, prec, 1.0, 1.0)
        assert (y.shape, y.dtype) == ((M, N), torch.bfloat16)


def test_fake_awq():
    with FakeTensorMode():
        x = torch.empty(2, 3072, dtype=torch.bfloat16)
        y = torch.ops.svdq.awq_gemv(x, torch.empty(18432, 1536, dtype=torch.uint8),
                                    torch.empty(18432, 48, dtype=torch.float16),
                                    torch.empty(18432, 48, dtype=torch.float16), None)
        assert (y.shape, y.dtype) == ((2, 18432), torch.bfloat16)


class _Block(torch.nn.Module):
    """Two quantized linears around a non-linearity, plus an AWQ projection of a
    conditioning vector: enough to show that the ops compose in one graph."""

    def __init__(self, prec):
        super().__init__()
        self.up = ops.SVDQLinear(256, 512, rank=16, precision=prec)
        self.down = ops.SVDQLinear(512, 256, rank=16, precision=prec)
        self.mod = ops.AWQLinear(256, 512)

    def forward(self, x, c):
        h = torch.nn.functional.gelu(self.up(x).float()).to(torch.bfloat16) * self.mod(c).unsqueeze(1)
        return self.down(h)


@pytest.mark.parametrize("prec", [sq.SVDQ_INT4, sq.SVDQ_NVFP4])
def test_export_full_graph(prec):
    m = _Block(prec)
    x = torch.zeros(2, 48, 256, dtype=torch.bfloat16)
    c = torch.zeros(2, 256, dtype=torch.bfloat16)
    ep = torch.export.export(m, (x, c), strict=True)
    targets = [n.target for n in ep.graph.nodes if n.op == "call_function"]
    assert targets.count(torch.ops.svdq.quantize_act.default) == 2
    assert targets.count(torch.ops.svdq.w4a4_gemm.default) == 2
    assert targets.count(torch.ops.svdq.awq_gemv.default) == 1
    out = [n for n in ep.graph.nodes if n.op == "output"][0].args[0][0].meta["val"]
    assert out.shape == (2, 48, 256) and out.dtype == torch.bfloat16


def test_fake_qkv():
    with FakeTensorMode():
        codes = torch.empty(4608, 1536, dtype=torch.uint8)
        y = torch.ops.svdq.w4a4_gemm_qkv_norm_rope(
            codes, torch.empty(4608, 48, dtype=torch.float16), torch.empty(9216, 1536, dtype=torch.uint8),
            torch.empty(9216, 48, dtype=torch.float16), torch.empty(4608, 32), torch.empty(9216, 32, dtype=torch.bfloat16),
            None, torch.empty(128, dtype=torch.bfloat16), torch.empty(128, dtype=torch.bfloat16),
            torch.empty(4608, 64, 2), 24, 128, 1e-6, sq.SVDQ_INT4, 1.0, 1.0)
        assert (y.shape, y.dtype) == ((4608, 9216), torch.bfloat16)


@pytest.mark.parametrize("ro", [0, 32])
def test_fake_gelu_quant(ro):
    M, K, N = 96, 256, 512
    with FakeTensorMode():
        codes = torch.empty(M, K // 2, dtype=torch.uint8)
        scales = torch.empty(M, K // 64, dtype=torch.float16)
        hc, hs, hx = torch.ops.svdq.w4a4_gemm_gelu_quant(
            codes, scales, torch.empty(N, K // 2, dtype=torch.uint8), torch.empty(N, K // 64, dtype=torch.float16),
            torch.empty(M, 16), torch.empty(N, 16, dtype=torch.bfloat16), None,
            torch.empty(N, dtype=torch.bfloat16), torch.empty(ro, N, dtype=torch.bfloat16) if ro else None,
            sq.SVDQ_INT4, 1.0, 1.0, 1.0)
        assert (hc.shape, hc.dtype) == ((M, N // 2), torch.uint8)
        assert (hs.shape, hs.dtype) == ((M, N // 64), torch.float16)
        assert (hx.shape, hx.dtype) == ((M, ro), torch.float32)


@pytest.mark.parametrize("prec", [sq.SVDQ_INT4, sq.SVDQ_NVFP4])
def test_export_mlp_full_graph(prec):
    m = ops.SVDQMLP(256, 1024, rank=16, precision=prec)
    x = torch.zeros(2, 48, 256, dtype=torch.bfloat16)
    ep = torch.export.export(m, (x,), strict=True)
    targets = [n.target for n in ep.graph.nodes if n.op == "call_function"]
    assert targets.count(torch.ops.svdq.quantize_act.default) == 1
    assert targets.count(torch.ops.svdq.w4a4_gemm_gelu_quant.default) == 1
    assert targets.count(torch.ops.svdq.w4a4_gemm.default) == 1
    out = [n for n in ep.graph.nodes if n.op == "output"][0].args[0][0].meta["val"]
    assert out.shape == (2, 48, 256) and out.dtype == torch.bfloat16


def test_fake_gemm_ws():
    with FakeTensorMode():
        codes = torch.empty(96, 256, dtype=torch.uint8)
        scales = torch.empty(96, 8, dtype=torch.float16)
        work = torch.empty(sq.GEMM_WORK_BYTES, dtype=torch.uint8)
        y = torch.ops.svdq.w4a4_gemm_ws(codes, scales, torch.empty(384, 256, dtype=torch.uint8),
                                        torch.empty(384, 8, dtype=torch.float16), None, None, None, work,
                                        sq.SVDQ_INT4, 1.0, 1.0)
        assert (y.shape, y.dtype) == ((96, 384), torch.bfloat16)


def test_fake_quantize_ws():
    with FakeTensorMode():
        x = torch.empty(96, 512, dtype=torch.bfloat16)
        work = torch.empty(sq.GEMM_WORK_BYTES, dtype=torch.uint8)
        for prec, sdt in ((sq.SVDQ_INT4, torch.float16), (sq.SVDQ_NVFP4, torch.uint8)):
            c, s, xl1 = torch.ops.svdq.quantize_act_ws(x, None, torch.empty(32, 512, dtype=torch.bfloat16), work,
                                                       prec, 1.0)
            assert c.shape == (96, 256) and s.dtype == sdt and s.shape == (96, 512 // sq.GROUP[prec])
            assert xl1.shape == (96, 32) and xl1.dtype == torch.float32


def test_export_with_workspace():
    # a layer given a workspace traces to quantize_act_ws + w4a4_gemm_ws, the
    # workspace a constant tensor of the graph
    m = ops.SVDQLinear(256, 384, rank=16)
    m.workspace = torch.zeros(sq.GEMM_WORK_BYTES, dtype=torch.uint8)
    ep = torch.export.export(m, (torch.zeros(2, 48, 256, dtype=torch.bfloat16),), strict=True)
    svdq_ops = [str(n.target) for n in ep.graph.nodes if n.op == "call_function" and "svdq" in str(n.target)]
    assert svdq_ops == ["svdq.quantize_act_ws.default", "svdq.w4a4_gemm_ws.default"]
