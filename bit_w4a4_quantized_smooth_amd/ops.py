"""torch custom ops over the C ABI, so that a model using the SVDQuant W4A4 and
AWQ W4A16 linears can be traced whole by torch.compile (fullgraph=True).

The pages say the quantized linear layers work under torch.compile ("Nunchaku
Lite", section "torch.compile"; blog "Nunchaku 4-bit inference in Diffusers",
"Benchmarks").  Here each library entry point becomes one opaque operator
(`svdq::quantize_act`, `svdq::quantize_act_ws`, `svdq::w4a4_gemm`, `svdq::w4a4_gemm_ws`,
`svdq::w4a4_gemm_qkv_norm_rope`, `svdq::w4a4_gemm_gelu_quant`, `svdq::awq_gemv`) with a fake
(meta) implementation that only computes output shapes and dtypes, so the
tracer never runs a kernel; the real implementation is the ctypes call into
libsvdq.so on the tensors' current stream.  Nothing here computes: every
arithmetic step stays in the library's kernels.

`SVDQLinear`, `SVDQMLP` and `AWQLinear` are nn.Modules holding the packed
layer tensors (as buffers) whose forward uses these operators; `SVDQMLP` is
the DiT MLP with the fused up-projection ("Nunchaku Lite", "Fused kernels":
the GELU-MLP fusion), three operators per call.  An SVDQLinear whose
`workspace` attribute holds a workspace from `gemm_workspace()` (one may serve
every layer that runs on the same stream) calls `svdq::quantize_act_ws` (a
call with fewer 32-row blocks than CUs spread over all of them) and
`svdq::w4a4_gemm_ws` (the GEMM grid's last partial round of tiles as K
slices).
"""
from __future__ import annotations

from typing import Optional, Tuple

import torch
from torch import Tensor

from . import (SVDQ_INT4, SVDQ_NVFP4, GROUP, awq_gemv, quantize_act, w4a4_gemm, w4a4_gemm_gelu_quant,
               w4a4_gemm_qkv_norm_rope)
from . import gemm_workspace  # noqa: F401  (re-exported for module users)

_SCALE_DTYPE = {SVDQ_INT4: torch.float16, SVDQ_NVFP4: torch.uint8}


@torch.library.custom_op("svdq::quantize_act", mutates_args=())
def quantize_act_op(x: Tensor, smooth: Optional[Tensor], l1t: Optional[Tensor], precision: int,
                    act_global_scale: float) -> Tuple[Tensor, Tensor, Tensor]:
    """svdq_quantize_act: returns (codes u8 [M, K/2], scales, xl1 fp32 [M, r]); r = 0 gives an
    empty xl1."""
    codes, scales, xl1 = quantize_act(precision, x, smooth, l1t, act_global_scale)
    if xl1 is None:
        xl1 = x.new_empty((x.shape[0], 0), dtype=torch.float32)
    return codes, scales, xl1


@quantize_act_op.register_fake
def _(x, smooth, l1t, precision, act_global_scale):
    M, K = x.shape
    r = 0 if l1t is None else l1t.shape[0]
    return (x.new_empty((M, K // 2), dtype=torch.uint8),
            x.new_empty((M, K // GROUP[precision]), dtype=_SCALE_DTYPE[precision]),
            x.new_empty((M, r), dtype=torch.float32))


@torch.library.custom_op("svdq::quantize_act_ws", mutates_args=("workspace",))
def quantize_act_ws_op(x: Tensor, smooth: Optional[Tensor], l1t: Optional[Tensor], workspace: Tensor,
                       precision: int, act_global_scale: float) -> Tuple[Tensor, Tensor, Tensor]:
    """svdq_quantize_act_ws: the outputs of svdq::quantize_act; `workspace` (u8
    [GEMM_WORK_BYTES], zero-filled once) is the one the stream's GEMMs use."""
    codes, scales, xl1 = quantize_act(precision, x, smooth, l1t, act_global_scale, workspace=workspace)
    if xl1 is None:
        xl1 = x.new_empty((x.shape[0], 0), dtype=torch.float32)
    return codes, scales, xl1


@quantize_act_ws_op.register_fake
def _(x, smooth, l1t, workspace, precision, act_global_scale):
    M, K = x.shape
    r = 0 if l1t is None else l1t.shape[0]
    return (x.new_empty((M, K // 2), dtype=torch.uint8),
            x.new_empty((M, K // GROUP[precision]), dtype=_SCALE_DTYPE[precision]),
            x.new_empty((M, r), dtype=torch.float32))


def _quant(x, smooth, l1t, precision, ags, workspace=None):
    if workspace is None:
        return torch.ops.svdq.quantize_act(x, smooth, l1t, precision, ags)
    return torch.ops.svdq.quantize_act_ws(x, smooth, l1t, workspace, precision, ags)


@torch.library.custom_op("svdq::w4a4_gemm", mutates_args=())
def w4a4_gemm_op(act_codes: Tensor, act_scales: Tensor, w_codes: Tensor, w_scales: Tensor,
                 xl1: Optional[Tensor], l2t: Optional[Tensor], bias: Optional[Tensor], precision: int,
                 act_global_scale: float, w_global_scale: float) -> Tensor:
    """svdq_w4a4_gemm: Y bf16 [M, N]."""
    if xl1 is not None and xl1.shape[1] == 0:
        xl1 = None
    return w4a4_gemm(precision, act_codes, act_scales, w_codes, w_scales, xl1, l2t, bias,
                     act_global_scale, w_global_scale)


@w4a4_gemm_op.register_fake
def _(act_codes, act_scales, w_codes, w_scales, xl1, l2t, bias, precision, act_global_scale, w_global_scale):
    return act_codes.new_empty((act_codes.shape[0], w_codes.shape[0]), dtype=torch.bfloat16)


@torch.library.custom_op("svdq::w4a4_gemm_ws", mutates_args=("workspace",))
def w4a4_gemm_ws_op(act_codes: Tensor, act_scales: Tensor, w_codes: Tensor, w_scales: Tensor,
                    xl1: Optional[Tensor], l2t: Optional[Tensor], bias: Optional[Tensor], workspace: Tensor,
                    precision: int, act_global_scale: float, w_global_scale: float) -> Tensor:
    """svdq_w4a4_gemm_ws: Y bf16 [M, N]; `workspace` (u8 [GEMM_WORK_BYTES], zero-filled once)
    receives the partial tiles of the split last round."""
    if xl1 is not None and xl1.shape[1] == 0:
        xl1 = None
    return w4a4_gemm(precision, act_codes, act_scales, w_codes, w_scales, xl1, l2t, bias,
                     act_global_scale, w_global_scale, workspace=workspace)


@w4a4_gemm_ws_op.register_fake
def _(act_codes, act_scales, w_codes, w_scales, xl1, l2t, bias, workspace, precision, act_global_scale,
      w_global_scale):
    return act_codes.new_empty((act_codes.shape[0], w_codes.shape[0]), dtype=torch.bfloat16)


def _gemm(codes, scales, w_codes, w_scales, xl1, l2t, bias, precision, ags, wgs, workspace=None):
    if workspace is None:
        return torch.ops.svdq.w4a4_gemm(codes, scales, w_codes, w_scales, xl1, l2t, bias, precision, ags, wgs)
    return torch.ops.svdq.w4a4_gemm_ws(codes, scales, w_codes, w_scales, xl1, l2t, bias, workspace, precision,
                                       ags, wgs)


@torch.library.custom_op("svdq::w4a4_gemm_qkv_norm_rope", mutates_args=())
def w4a4_gemm_qkv_op(act_codes: Tensor, act_scales: Tensor, w_codes: Tensor, w_scales: Tensor,
                     xl1: Optional[Tensor], l2t: Optional[Tensor], bias: Optional[Tensor], norm_q: Tensor,
                     norm_k: Tensor, rope: Optional[Tensor], heads: int, head_dim: int, eps: float,
                     precision: int, act_global_scale: float, w_global_scale: float) -> Tensor:
    """svdq_w4a4_gemm_qkv_norm_rope: Y bf16 [M, 3 * heads * head_dim]."""
    if xl1 is not None and xl1.shape[1] == 0:
        xl1 = None
    return w4a4_gemm_qkv_norm_rope(precision, act_codes, act_scales, w_codes, w_scales, xl1, l2t, bias, heads,
                                   head_dim, norm_q, norm_k, eps, rope, act_global_scale, w_global_scale)


@w4a4_gemm_qkv_op.register_fake
def _(act_codes, act_scales, w_codes, w_scales, xl1, l2t, bias, norm_q, norm_k, rope, heads, head_dim, eps,
      precision, act_global_scale, w_global_scale):
    return act_codes.new_empty((act_codes.shape[0], 3 * heads * head_dim), dtype=torch.bfloat16)


@torch.library.custom_op("svdq::w4a4_gemm_gelu_quant", mutates_args=())
def w4a4_gemm_gelu_quant_op(act_codes: Tensor, act_scales: Tensor, w_codes: Tensor, w_scales: Tensor,
                            xl1: Optional[Tensor], l2t: Optional[Tensor], bias: Optional[Tensor],
                            smooth_out: Optional[Tensor], l1t_out: Optional[Tensor], precision: int,
                            act_global_scale: float, w_global_scale: float,
                            out_global_scale: float) -> Tuple[Tensor, Tensor, Tensor]:
    """svdq_w4a4_gemm_gelu_quant: the MLP up-projection, GELU and the down
    projection's activation quantization; returns (codes u8 [M, N/2], scales
    [M, N/G], xl1 fp32 [M, r_out]), r_out = 0 giving an empty xl1."""
    if xl1 is not None and xl1.shape[1] == 0:
        xl1 = None
    codes, scales, xo = w4a4_gemm_gelu_quant(act_codes, act_scales, w_codes, w_scales, xl1, l2t, bias,
                                             smooth_out, l1t_out, precision=precision,
                                             act_global_scale=act_global_scale, w_global_scale=w_global_scale,
                                             out_global_scale=out_global_scale)
    if xo is None:
        xo = act_codes.new_empty((act_codes.shape[0], 0), dtype=torch.float32)
    return codes, scales, xo


@w4a4_gemm_gelu_quant_op.register_fake
def _(act_codes, act_scales, w_codes, w_scales, xl1, l2t, bias, smooth_out, l1t_out, precision,
      act_global_scale, w_global_scale, out_global_scale):
    M, N = act_codes.shape[0], w_codes.shape[0]
    ro = 0 if l1t_out is None else l1t_out.shape[0]
    return (act_codes.new_empty((M, N // 2), dtype=torch.uint8),
            act_codes.new_empty((M, N // GROUP[precision]), dtype=_SCALE_DTYPE[precision]),
            act_codes.new_empty((M, ro), dtype=torch.float32))


@torch.library.custom_op("svdq::awq_gemv", mutates_args=())
def awq_gemv_op(x: Tensor, w_codes: Tensor, w_scales: Tensor, w_zeros: Tensor, bias: Optional[Tensor]) -> Tensor:
    """awq_w4a16_gemv: y bf16 [M, N]."""
    return awq_gemv(x, w_codes, w_scales, w_zeros, bias)


@awq_gemv_op.register_fake
def _(x, w_codes, w_scales, w_zeros, bias):
    return x.new_empty((x.shape[0], w_codes.shape[0]), dtype=torch.bfloat16)


def svdq_linear(x: Tensor, smooth: Optional[Tensor], l1t: Optional[Tensor], w_codes: Tensor, w_scales: Tensor,
                l2t: Optional[Tensor], bias: Optional[Tensor], precision: int = SVDQ_INT4,
                act_global_scale: float = 1.0, w_global_scale: float = 1.0,
                workspace: Optional[Tensor] = None) -> Tensor:
    """The SVDQuant linear as two traceable operators; x may have any leading shape.  With a
    `workspace` (gemm_workspace()) the operators are svdq::quantize_act_ws and svdq::w4a4_gemm_ws."""
    lead = x.shape[:-1]
    x2 = x.reshape(-1, x.shape[-1])
    codes, scales, xl1 = _quant(x2, smooth, l1t, precision, act_global_scale, workspace)
    y = _gemm(codes, scales, w_codes, w_scales, xl1, l2t, bias, precision, act_global_scale, w_global_scale,
              workspace)
    return y.reshape(*lead, w_codes.shape[0])


class SVDQLinear(torch.nn.Module):
    """A linear layer in SVDQuant W4A4 form ([Lite] "NunchakuLiteQuantizationConfig":
    precision, group size, rank): smoothing factor, rank-r low-rank branch in bf16,
    4-bit residual weight with per-group scales.  Tensors use the C ABI's layouts
    (nn.Linear orientation: codes [N, K/2], l1t = L1^T [r, K], l2t = L2^T [N, r])."""

    def __init__(self, in_features: int, out_features: int, rank: int = 32, precision: int = SVDQ_INT4,
                 bias: bool = True, device=None):
        super().__init__()
        G = GROUP[precision]
        self.precision, self.rank = precision, rank
        self.in_features, self.out_features = in_features, out_features
        kw = dict(device=device)
        self.register_buffer("smooth", torch.ones(in_features, dtype=torch.bfloat16, **kw))
        self.register_buffer("w_codes", torch.zeros(out_features, in_features // 2, dtype=torch.uint8, **kw))
        self.register_buffer("w_scales", torch.zeros(out_features, in_features // G, dtype=_SCALE_DTYPE[precision], **kw))
        self.register_buffer("l1t", torch.zeros(rank, in_features, dtype=torch.bfloat16, **kw) if rank else None)
        self.register_buffer("l2t", torch.zeros(out_features, rank, dtype=torch.bfloat16, **kw) if rank else None)
        self.register_buffer("bias", torch.zeros(out_features, dtype=torch.bfloat16, **kw) if bias else None)
        self.act_global_scale = 1.0  # NVFP4: static, calibrated offline
        self.w_global_scale = 1.0
        # optional GEMM workspace (gemm_workspace()), shared by the layers of one stream:
        # an attribute, not a buffer, so that one 16 MiB workspace serves them all
        self.workspace: Optional[Tensor] = None

    def forward(self, x: Tensor) -> Tensor:
        return svdq_linear(x, self.smooth, self.l1t, self.w_codes, self.w_scales, self.l2t, self.bias,
                           self.precision, self.act_global_scale, self.w_global_scale, self.workspace)


class SVDQMLP(torch.nn.Module):
    """The DiT MLP dim -> hidden -> dim in SVDQuant W4A4 form (int4 or nvfp4),
    with the up-projection, GELU and the down projection's activation
    quantization (and its low-rank input XL1) fused in one kernel:
    quantize_act, then w4a4_gemm_gelu_quant, then w4a4_gemm.  `up` and `down`
    hold the two layers' tensors as SVDQLinear does; the down layer's smoothing
    factor, L1^T and activation global scale are consumed by the fused kernel,
    its codes, scales, L2^T and bias by the GEMM."""

    def __init__(self, dim: int, hidden: int, rank: int = 32, precision: int = SVDQ_INT4, bias: bool = True,
                 device=None):
        super().__init__()
        self.precision = precision
        self.up = SVDQLinear(dim, hidden, rank=rank, precision=precision, bias=bias, device=device)
        self.down = SVDQLinear(hidden, dim, rank=rank, precision=precision, bias=bias, device=device)

    def forward(self, x: Tensor) -> Tensor:
        lead = x.shape[:-1]
        x2 = x.reshape(-1, x.shape[-1])
        up, down, p = self.up, self.down, self.precision
        codes, scales, xl1 = _quant(x2, up.smooth, up.l1t, p, up.act_global_scale, up.workspace)
        hc, hs, hx = torch.ops.svdq.w4a4_gemm_gelu_quant(codes, scales, up.w_codes, up.w_scales, xl1, up.l2t,
                                                         up.bias, down.smooth, down.l1t, p, up.act_global_scale,
                                                         up.w_global_scale, down.act_global_scale)
        y = _gemm(hc, hs, down.w_codes, down.w_scales, hx, down.l2t, down.bias, p, down.act_global_scale,
                  down.w_global_scale, down.workspace)
        return y.reshape(*lead, down.out_features)


class AWQLinear(torch.nn.Module):
    """A linear layer in AWQ W4A16 form (int4 weight-only, group 64, unsigned codes with
    fp16 scale and zero-point per (row, group))."""

    def __init__(self, in_features: int, out_features: int, bias: bool = True, device=None):
        super().__init__()
        kw = dict(device=device)
        self.register_buffer("w_codes", torch.zeros(out_features, in_features // 2, dtype=torch.uint8, **kw))
        self.register_buffer("w_scales", torch.zeros(out_features, in_features // 64, dtype=torch.float16, **kw))
        self.register_buffer("w_zeros", torch.zeros(out_features, in_features // 64, dtype=torch.float16, **kw))
        self.register_buffer("bias", torch.zeros(out_features, dtype=torch.bfloat16, **kw) if bias else None)

    def forward(self, x: Tensor) -> Tensor:
        lead = x.shape[:-1]
        y = torch.ops.svdq.awq_gemv(x.reshape(-1, x.shape[-1]), self.w_codes, self.w_scales, self.w_zeros, self.bias)
        return y.reshape(*lead, self.w_codes.shape[0])
