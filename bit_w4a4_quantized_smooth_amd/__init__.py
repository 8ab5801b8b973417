"""Python binding of libsvdq.so: the SVDQuant W4A4 linear and the AWQ W4A16
linear as gfx950 HIP kernels behind a C ABI (include/svdq.h).

This module only marshals arguments: torch tensors supply device pointers and
the current HIP stream; every step of the computation runs in the library's
kernels.  There is no fallback: if libsvdq.so is missing or the device is not
gfx950, every call raises.

Tensor conventions (all on the GPU, contiguous):
  bf16 tensors are torch.bfloat16; fp16 scales torch.float16; E4M3 scales and
  packed 4-bit codes torch.uint8; xl1 and psums float32 / int32.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsvdq.so")

SVDQ_INT4, SVDQ_NVFP4 = 0, 1
GROUP = {SVDQ_INT4: 64, SVDQ_NVFP4: 16}
_STATUS = {0: "SVDQ_OK", 1: "SVDQ_ERR_INVALID_ARG", 2: "SVDQ_ERR_UNSUPPORTED",
           3: "SVDQ_ERR_ALIGNMENT", 4: "SVDQ_ERR_DEVICE"}

EXPORTS = ["svdq_quantize_act", "svdq_w4a4_gemm", "svdq_w4a4_gemm_qkv_norm_rope", "svdq_w4a4_gemm_gelu_quant",
           "awq_w4a16_gemv", "svdq_calibrate_smooth", "svdq_lowrank_workspace_bytes", "svdq_lowrank_decompose",
           "svdq_quantize_weight", "awq_quantize_weight",
           "svdq_w4a4_group_psums", "svdq_last_error", "svdq_abi_version", "svdq_test_set_arch_override"]


class SvdqError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{_STATUS.get(status, status)}: {msg}")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """Loads libsvdq.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -c 'import __graft_entry__ as g; g.build()'`")
        L = ctypes.CDLL(LIB_PATH)
        i64, vp, f32, i32 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_float, ctypes.c_int
        L.svdq_quantize_act.argtypes = [i32, i32, i32, i64, i64, vp, vp, vp, f32, vp, vp, vp, vp]
        L.svdq_w4a4_gemm.argtypes = [i32, i32, i32, i64, i64, i64, vp, vp, f32, vp, vp, f32, vp, vp,
                                     vp, vp, vp]
        L.svdq_w4a4_gemm_qkv_norm_rope.argtypes = [i32, i32, i32, i64, i32, i32, i64, vp, vp, f32, vp, vp,
                                                   f32, vp, vp, vp, vp, vp, f32, vp, i64, vp, vp]
        L.svdq_w4a4_gemm_gelu_quant.argtypes = [i32, i32, i32, i64, i64, i64, vp, vp, f32, vp, vp, f32, vp, vp,
                                                vp, vp, vp, i32, vp, vp, vp, vp]
        L.awq_w4a16_gemv.argtypes = [i32, i64, i64, i64, vp, vp, vp, vp, vp, vp, vp]
        L.svdq_calibrate_smooth.argtypes = [i64, i64, i64, vp, vp, vp, vp]
        L.svdq_lowrank_workspace_bytes.argtypes = [i64, i64, i32, i32]
        L.svdq_lowrank_workspace_bytes.restype = i64
        L.svdq_lowrank_decompose.argtypes = [i64, i64, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, i64, vp]
        L.svdq_quantize_weight.argtypes = [i32, i32, i64, i64, vp, f32, vp, vp, vp]
        L.awq_quantize_weight.argtypes = [i32, i64, i64, vp, vp, vp, vp, vp]
        L.svdq_w4a4_group_psums.argtypes = [i32, i32, i64, i64, i64, vp, vp, vp, vp]
        for f in ("svdq_quantize_act", "svdq_w4a4_gemm", "svdq_w4a4_gemm_qkv_norm_rope",
                  "svdq_w4a4_gemm_gelu_quant", "awq_w4a16_gemv", "svdq_w4a4_group_psums", "svdq_calibrate_smooth",
                  "svdq_lowrank_decompose", "svdq_quantize_weight", "awq_quantize_weight"):
            getattr(L, f).restype = i32
        L.svdq_last_error.restype = ctypes.c_char_p
        L.svdq_abi_version.restype = i32
        L.svdq_test_set_arch_override.argtypes = [ctypes.c_char_p]
        L.svdq_test_set_arch_override.restype = None
        _lib = L
    return _lib


def _check(status: int) -> None:
    if status != 0:
        raise SvdqError(status, lib().svdq_last_error().decode())


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def quantize_act(precision: int, x, smooth=None, l1t=None, act_global_scale: float = 1.0,
                 out=None, stream=None):
    """svdq_quantize_act.  x: bf16 [M, K]; smooth: bf16 [K] or None; l1t: bf16 [r, K]
    or None.  Returns (codes u8 [M, K/2], scales, xl1 fp32 [M, r] or None); `out`
    may supply that triple preallocated."""
    M, K = x.shape
    G = GROUP.get(precision, 64)
    r = 0 if l1t is None else l1t.shape[0]
    if out is None:
        codes = torch.empty((M, K // 2), dtype=torch.uint8, device=x.device)
        scales = (torch.empty((M, K // G), dtype=torch.float16, device=x.device) if precision == SVDQ_INT4
                  else torch.empty((M, K // G), dtype=torch.uint8, device=x.device))
        xl1 = torch.empty((M, r), dtype=torch.float32, device=x.device) if r else None
    else:
        codes, scales, xl1 = out
    _check(lib().svdq_quantize_act(precision, G, r, M, K, _ptr(x), _ptr(smooth), _ptr(l1t),
                                   float(act_global_scale), _ptr(codes), _ptr(scales), _ptr(xl1),
                                   _stream(stream)))
    return codes, scales, xl1


def w4a4_gemm(precision: int, act_codes, act_scales, w_codes, w_scales, xl1=None, l2t=None,
              bias=None, act_global_scale: float = 1.0, w_global_scale: float = 1.0, out=None,
              stream=None):
    """svdq_w4a4_gemm.  Returns Y bf16 [M, N]."""
    M, K = act_codes.shape[0], act_codes.shape[1] * 2
    N = w_codes.shape[0]
    G = GROUP.get(precision, 64)
    r = 0 if l2t is None else l2t.shape[1]
    y = out if out is not None else torch.empty((M, N), dtype=torch.bfloat16, device=act_codes.device)
    _check(lib().svdq_w4a4_gemm(precision, G, r, M, N, K, _ptr(act_codes), _ptr(act_scales),
                                float(act_global_scale), _ptr(w_codes), _ptr(w_scales),
                                float(w_global_scale), _ptr(xl1), _ptr(l2t), _ptr(bias), _ptr(y),
                                _stream(stream)))
    return y


def w4a4_gemm_qkv_norm_rope(precision: int, act_codes, act_scales, w_codes, w_scales, xl1, l2t, bias,
                            heads: int, head_dim: int, norm_q, norm_k, eps: float, rope=None,
                            act_global_scale: float = 1.0, w_global_scale: float = 1.0, out=None,
                            stream=None):
    """svdq_w4a4_gemm_qkv_norm_rope: the fused attention projection.  w_codes holds the Q, K
    and V weights concatenated along N (= 3 * heads * head_dim); rope is fp32
    [S, head_dim/2, 2] (cos, sin) or None.  Returns Y bf16 [M, N]."""
    M, K = act_codes.shape[0], act_codes.shape[1] * 2
    N = w_codes.shape[0]
    G = GROUP.get(precision, 64)
    r = 0 if l2t is None else l2t.shape[1]
    rope_rows = 0 if rope is None else rope.shape[0]
    y = out if out is not None else torch.empty((M, N), dtype=torch.bfloat16, device=act_codes.device)
    _check(lib().svdq_w4a4_gemm_qkv_norm_rope(
        precision, G, r, M, heads, head_dim, K, _ptr(act_codes), _ptr(act_scales), float(act_global_scale),
        _ptr(w_codes), _ptr(w_scales), float(w_global_scale), _ptr(xl1), _ptr(l2t), _ptr(bias), _ptr(norm_q),
        _ptr(norm_k), float(eps), _ptr(rope), rope_rows, _ptr(y), _stream(stream)))
    return y


def w4a4_gemm_gelu_quant(act_codes, act_scales, w_codes, w_scales, xl1, l2t, bias, smooth_out=None,
                         l1t_out=None, out=None, stream=None):
    """svdq_w4a4_gemm_gelu_quant (int4): the MLP up-projection with GELU and the down
    projection's quantization fused.  Returns (codes u8 [M, N/2], scales fp16 [M, N/64],
    xl1 fp32 [M, r_out] or None); `out` may supply that triple preallocated."""
    M, K = act_codes.shape[0], act_codes.shape[1] * 2
    N = w_codes.shape[0]
    r = 0 if l2t is None else l2t.shape[1]
    ro = 0 if l1t_out is None else l1t_out.shape[0]
    if out is None:
        dev = act_codes.device
        out = (torch.empty((M, N // 2), dtype=torch.uint8, device=dev),
               torch.empty((M, N // 64), dtype=torch.float16, device=dev),
               torch.empty((M, ro), dtype=torch.float32, device=dev) if ro else None)
    codes, scales, xo = out
    _check(lib().svdq_w4a4_gemm_gelu_quant(
        SVDQ_INT4, 64, r, M, N, K, _ptr(act_codes), _ptr(act_scales), 1.0, _ptr(w_codes), _ptr(w_scales), 1.0,
        _ptr(xl1), _ptr(l2t), _ptr(bias), _ptr(smooth_out), _ptr(l1t_out), ro, _ptr(codes), _ptr(scales),
        _ptr(xo), _stream(stream)))
    return codes, scales, xo


def calibrate_smooth(x_cal, w, out=None, stream=None):
    """svdq_calibrate_smooth: lambda bf16 [K] from calibration activations and the dense weight."""
    Mc, K = x_cal.shape
    N = w.shape[0]
    lam = out if out is not None else torch.empty(K, dtype=torch.bfloat16, device=w.device)
    _check(lib().svdq_calibrate_smooth(Mc, N, K, _ptr(x_cal), _ptr(w), _ptr(lam), _stream(stream)))
    return lam


def lowrank_decompose(w, smooth, omega, rank: int, iters: int = 4, stream=None):
    """svdq_lowrank_decompose: returns (l1t bf16 [rank, K], l2t bf16 [N, rank], residual fp32 [N, K]).
    omega: fp32 [K, rank + oversample] test matrix."""
    N, K = w.shape
    p = omega.shape[1]
    nbytes = lib().svdq_lowrank_workspace_bytes(N, K, rank, p - rank)
    if nbytes < 0:
        raise SvdqError(2, f"unsupported decomposition sizes N={N} K={K} rank={rank} p={p}")
    dev = w.device
    work = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    l1t = torch.empty((rank, K), dtype=torch.bfloat16, device=dev)
    l2t = torch.empty((N, rank), dtype=torch.bfloat16, device=dev)
    res = torch.empty((N, K), dtype=torch.float32, device=dev)
    _check(lib().svdq_lowrank_decompose(N, K, rank, p - rank, iters, _ptr(w), _ptr(smooth), _ptr(omega), _ptr(l1t),
                                        _ptr(l2t), _ptr(res), _ptr(work), nbytes, _stream(stream)))
    return l1t, l2t, res


def quantize_weight(precision: int, residual, w_global_scale: float = 1.0, out=None, stream=None):
    """svdq_quantize_weight: (codes u8 [N, K/2], scales) of an fp32 residual [N, K]."""
    N, K = residual.shape
    G = GROUP.get(precision, 64)
    if out is None:
        out = (torch.empty((N, K // 2), dtype=torch.uint8, device=residual.device),
               torch.empty((N, K // G), dtype=torch.float16 if precision == SVDQ_INT4 else torch.uint8,
                           device=residual.device))
    _check(lib().svdq_quantize_weight(precision, G, N, K, _ptr(residual), float(w_global_scale), _ptr(out[0]),
                                      _ptr(out[1]), _stream(stream)))
    return out


def awq_quantize_weight(w, out=None, stream=None):
    """awq_quantize_weight: (codes u8 [N, K/2], scales fp16 [N, K/64], zeros fp16 [N, K/64])."""
    N, K = w.shape
    if out is None:
        dev = w.device
        out = (torch.empty((N, K // 2), dtype=torch.uint8, device=dev),
               torch.empty((N, K // 64), dtype=torch.float16, device=dev),
               torch.empty((N, K // 64), dtype=torch.float16, device=dev))
    _check(lib().awq_quantize_weight(64, N, K, _ptr(w), _ptr(out[0]), _ptr(out[1]), _ptr(out[2]), _stream(stream)))
    return out


def group_psums(precision: int, act_codes, w_codes, out=None, stream=None):
    """svdq_w4a4_group_psums (test support).  Returns [M, N, K/G] int32 (int4) or fp32 (nvfp4)."""
    M, K = act_codes.shape[0], act_codes.shape[1] * 2
    N = w_codes.shape[0]
    G = GROUP.get(precision, 64)
    if out is None:
        out = torch.empty((M, N, K // G), dtype=torch.int32 if precision == SVDQ_INT4 else torch.float32,
                          device=act_codes.device)
    _check(lib().svdq_w4a4_group_psums(precision, G, M, N, K, _ptr(act_codes), _ptr(w_codes),
                                       _ptr(out), _stream(stream)))
    return out


def awq_gemv(x, w_codes, w_scales, w_zeros, bias=None, out=None, stream=None, group_size: int = 64):
    """awq_w4a16_gemv.  x bf16 [M, K]; returns Y bf16 [M, N]."""
    M, K = x.shape
    N = w_codes.shape[0]
    y = out if out is not None else torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    _check(lib().awq_w4a16_gemv(group_size, M, N, K, _ptr(x), _ptr(w_codes), _ptr(w_scales),
                                _ptr(w_zeros), _ptr(bias), _ptr(y), _stream(stream)))
    return y


def svdq_linear(precision: int, x, smooth, l1t, w_codes, w_scales, l2t, bias,
                act_global_scale: float = 1.0, w_global_scale: float = 1.0, stream=None):
    """The whole SVDQuant linear: quantize (+ X.L1) then the 4-bit GEMM (+ low-rank up, bias)."""
    codes, scales, xl1 = quantize_act(precision, x, smooth, l1t, act_global_scale, stream=stream)
    return w4a4_gemm(precision, codes, scales, w_codes, w_scales, xl1, l2t, bias,
                     act_global_scale, w_global_scale, stream=stream)


def abi_version() -> int:
    return lib().svdq_abi_version()


def set_arch_override(arch):
    """Test hook: make the architecture check see `arch` (None restores the device's)."""
    lib().svdq_test_set_arch_override(None if arch is None else arch.encode())
