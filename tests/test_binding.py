"""The Python binding rejects, with ValueError and before any pointer reaches
the library, tensors of the wrong dtype, shape, layout or device: a host
tensor would hand a host pointer to a kernel, an undersized output would be
written out of bounds and a mismatched operand read out of bounds.  These
tests run on a host without a GPU and launch nothing."""
import pytest
import torch

import bit_w4a4_quantized_smooth_amd as sq

bf16, f16, f32, u8, i32 = torch.bfloat16, torch.float16, torch.float32, torch.uint8, torch.int32


def z(*shape, dtype=u8):
    return torch.zeros(shape, dtype=dtype)


def gemm_inputs(M=32, N=128, K=256, r=16, prec=sq.SVDQ_INT4):
    G = sq.GROUP[prec]
    sd = f16 if prec == sq.SVDQ_INT4 else u8
    return dict(act_codes=z(M, K // 2), act_scales=z(M, K // G, dtype=sd), w_codes=z(N, K // 2),
                w_scales=z(N, K // G, dtype=sd), xl1=z(M, r, dtype=f32), l2t=z(N, r, dtype=bf16),
                bias=z(N, dtype=bf16))


def call_gemm(prec=sq.SVDQ_INT4, out=None, **kw):
    a = gemm_inputs(prec=prec)
    a.update(kw)
    return sq.w4a4_gemm(prec, a["act_codes"], a["act_scales"], a["w_codes"], a["w_scales"], a["xl1"], a["l2t"],
                        a["bias"], out=out)


def test_host_tensors_are_rejected():
    with pytest.raises(ValueError, match="not on a GPU"):
        sq.quantize_act(sq.SVDQ_INT4, z(8, 64, dtype=bf16))
    with pytest.raises(ValueError, match="not on a GPU"):
        call_gemm()
    with pytest.raises(ValueError, match="not on a GPU"):
        sq.awq_gemv(z(2, 128, dtype=bf16), z(64, 64), z(64, 2, dtype=f16), z(64, 2, dtype=f16))
    with pytest.raises(ValueError, match="not on a GPU"):
        sq.group_psums(sq.SVDQ_INT4, z(8, 32), z(128, 32))


def test_dtypes_are_checked():
    with pytest.raises(ValueError, match="x must be torch.bfloat16"):
        sq.quantize_act(sq.SVDQ_INT4, z(8, 64, dtype=f32))
    with pytest.raises(ValueError, match="act_scales must be torch.float16"):
        call_gemm(act_scales=z(32, 4, dtype=f32))
    with pytest.raises(ValueError, match="w_scales must be torch.uint8"):
        call_gemm(prec=sq.SVDQ_NVFP4, w_scales=z(128, 16, dtype=f16))
    with pytest.raises(ValueError, match="w_scales must be torch.float16"):
        sq.awq_gemv(z(2, 128, dtype=bf16), z(64, 64), z(64, 2, dtype=f32), z(64, 2, dtype=f16))
    with pytest.raises(ValueError, match="residual must be torch.float32"):
        sq.quantize_weight(sq.SVDQ_INT4, z(64, 128, dtype=bf16))


def test_shapes_must_agree():
    # K of the weight operands, rank of the low-rank operands, N of bias and l2t
    with pytest.raises(ValueError, match="w_codes must have shape"):
        call_gemm(w_codes=z(128, 64))
    with pytest.raises(ValueError, match="w_scales must have shape"):
        call_gemm(w_scales=z(128, 3, dtype=f16))
    with pytest.raises(ValueError, match="xl1 must have shape"):
        call_gemm(xl1=z(32, 32, dtype=f32))
    with pytest.raises(ValueError, match="bias must have shape"):
        call_gemm(bias=z(64, dtype=bf16))
    with pytest.raises(ValueError, match="xl1 is required"):
        call_gemm(xl1=None)
    with pytest.raises(ValueError, match="l1t must have shape"):
        sq.quantize_act(sq.SVDQ_INT4, z(8, 64, dtype=bf16), None, z(16, 128, dtype=bf16))
    with pytest.raises(ValueError, match="smooth must have shape"):
        sq.quantize_act(sq.SVDQ_INT4, z(8, 64, dtype=bf16), z(32, dtype=bf16))
    with pytest.raises(ValueError, match="w_zeros must have shape"):
        sq.awq_gemv(z(2, 128, dtype=bf16), z(64, 64), z(64, 2, dtype=f16), z(64, 1, dtype=f16))
    with pytest.raises(ValueError, match="norm_q must have shape"):
        a = gemm_inputs(N=384)
        sq.w4a4_gemm_qkv_norm_rope(sq.SVDQ_INT4, a["act_codes"], a["act_scales"], a["w_codes"], a["w_scales"],
                                   a["xl1"], a["l2t"], a["bias"], 1, 128, z(64, dtype=bf16), z(128, dtype=bf16),
                                   1e-6)
    with pytest.raises(ValueError, match="w_codes must have shape"):  # N = 3 * heads * head_dim
        a = gemm_inputs(N=384)
        sq.w4a4_gemm_qkv_norm_rope(sq.SVDQ_INT4, a["act_codes"], a["act_scales"], a["w_codes"], a["w_scales"],
                                   a["xl1"], a["l2t"], a["bias"], 2, 128, z(128, dtype=bf16), z(128, dtype=bf16),
                                   1e-6)


def test_undersized_outputs_are_rejected():
    with pytest.raises(ValueError, match="y must have shape"):
        call_gemm(out=z(32, 64, dtype=bf16))
    with pytest.raises(ValueError, match="codes must have shape"):
        sq.quantize_act(sq.SVDQ_INT4, z(8, 64, dtype=bf16), out=(z(8, 16), z(8, 1, dtype=f16), None))
    with pytest.raises(ValueError, match="xl1_out must have shape"):
        a = gemm_inputs()
        sq.w4a4_gemm_gelu_quant(a["act_codes"], a["act_scales"], a["w_codes"], a["w_scales"], a["xl1"], a["l2t"],
                                a["bias"], None, z(16, 128, dtype=bf16),
                                out=(z(32, 64), z(32, 2, dtype=f16), z(32, 8, dtype=f32)))
    with pytest.raises(ValueError, match="psums must have shape"):
        sq.group_psums(sq.SVDQ_INT4, z(8, 32), z(128, 32), out=z(8, 128, 2, dtype=i32))


def test_layout_and_types():
    with pytest.raises(ValueError, match="contiguous"):
        sq.quantize_act(sq.SVDQ_INT4, z(64, 8, dtype=bf16).t())
    with pytest.raises(ValueError, match="2-D torch.Tensor"):
        sq.quantize_act(sq.SVDQ_INT4, z(64, dtype=bf16))
    with pytest.raises(ValueError, match="must be a torch.Tensor"):
        call_gemm(bias=[0.0] * 128)


def test_gemm_workspace_is_checked():
    a = gemm_inputs()
    args = (sq.SVDQ_INT4, a["act_codes"], a["act_scales"], a["w_codes"], a["w_scales"], a["xl1"], a["l2t"], a["bias"])
    with pytest.raises(ValueError, match="workspace must have shape"):
        sq.w4a4_gemm(*args, workspace=z(1024))
    with pytest.raises(ValueError, match="workspace must be torch.uint8"):
        sq.w4a4_gemm(*args, workspace=z(sq.GEMM_WORK_BYTES // 4, dtype=f32))
    with pytest.raises(ValueError, match="not on a GPU"):
        sq.w4a4_gemm(*args, workspace=z(sq.GEMM_WORK_BYTES))
