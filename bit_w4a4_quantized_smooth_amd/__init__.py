"""Python binding of libsvdq.so: the SVDQuant W4A4 linear and the AWQ W4A16
linear as gfx950 HIP kernels behind a C ABI (include/svdq.h).

This module only marshals arguments: torch tensors supply device pointers and
the current HIP stream; every step of the computation runs in the library's
kernels.  There is no fallback: if libsvdq.so is missing or the device is not
gfx950, every call raises.

Tensor conventions (all on one GPU, contiguous):
  bf16 tensors are torch.bfloat16; fp16 scales torch.float16; E4M3 scales and
  packed 4-bit codes torch.uint8; xl1 and psums float32 / int32.  Every wrapper
  checks dtypes, shapes, contiguity and the device of its tensors (ValueError)
  before a pointer reaches the library; the library then checks sizes, limits,
  alignment and aliasing (SvdqError).
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# SVDQ_LIB: another build of the library (the sanitizer test loads a
# host-only ASan/UBSan build of the C ABI layer this way)
LIB_PATH = os.environ.get("SVDQ_LIB") or os.path.join(_HERE, "libsvdq.so")

SVDQ_INT4, SVDQ_NVFP4 = 0, 1
GROUP = {SVDQ_INT4: 64, SVDQ_NVFP4: 16}
_STATUS = {0: "SVDQ_OK", 1: "SVDQ_ERR_INVALID_ARG", 2: "SVDQ_ERR_UNSUPPORTED",
           3: "SVDQ_ERR_ALIGNMENT", 4: "SVDQ_ERR_DEVICE"}

# SVDQ_GEMM_WORK_BYTES: size of svdq_w4a4_gemm_ws's workspace
GEMM_WORK_BYTES = 16 * 1024 * 1024 + 4096

EXPORTS = ["svdq_quantize_act", "svdq_quantize_act_ws", "svdq_w4a4_gemm", "svdq_w4a4_gemm_ws",
           "svdq_w4a4_gemm_qkv_norm_rope", "svdq_w4a4_gemm_qkv_norm_rope_ws", "svdq_w4a4_gemm_gelu_quant",
           "awq_w4a16_gemv", "svdq_quantize_act_awq_gemv", "svdq_calibrate_smooth",
           "svdq_lowrank_workspace_bytes", "svdq_lowrank_decompose", "svdq_lowrank_decompose_noalloc",
           "svdq_quantize_weight", "awq_quantize_weight",
           "svdq_w4a4_group_psums", "svdq_last_error", "svdq_abi_version", "svdq_test_set_arch_override",
           "svdq_test_set_no_ksplit"]


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
        L.svdq_quantize_act_ws.argtypes = [i32, i32, i32, i64, i64, vp, vp, vp, f32, vp, vp, vp, vp, i64, vp]
        L.svdq_w4a4_gemm.argtypes = [i32, i32, i32, i64, i64, i64, vp, vp, f32, vp, vp, f32, vp, vp,
                                     vp, vp, vp]
        L.svdq_w4a4_gemm_ws.argtypes = [i32, i32, i32, i64, i64, i64, vp, vp, f32, vp, vp, f32, vp, vp,
                                        vp, vp, vp, i64, vp]
        L.svdq_w4a4_gemm_qkv_norm_rope.argtypes = [i32, i32, i32, i64, i32, i32, i64, vp, vp, f32, vp, vp,
                                                   f32, vp, vp, vp, vp, vp, f32, vp, i64, vp, vp]
        L.svdq_w4a4_gemm_qkv_norm_rope_ws.argtypes = [i32, i32, i32, i64, i32, i32, i64, vp, vp, f32, vp, vp,
                                                      f32, vp, vp, vp, vp, vp, f32, vp, i64, vp, vp, i64, vp]
        L.svdq_w4a4_gemm_gelu_quant.argtypes = [i32, i32, i32, i64, i64, i64, vp, vp, f32, vp, vp, f32, vp, vp,
                                                vp, vp, vp, i32, f32, vp, vp, vp, vp]
        L.awq_w4a16_gemv.argtypes = [i32, i64, i64, i64, vp, vp, vp, vp, vp, vp, vp]
        L.svdq_quantize_act_awq_gemv.argtypes = [i32, i32, i32, i64, i64, vp, vp, vp, f32, vp, vp, vp,
                                                 i32, i64, i64, i64, vp, vp, vp, vp, vp, vp, vp]
        L.svdq_calibrate_smooth.argtypes = [i64, i64, i64, vp, vp, vp, vp]
        L.svdq_lowrank_workspace_bytes.argtypes = [i64, i64, i32, i32]
        L.svdq_lowrank_workspace_bytes.restype = i64
        L.svdq_lowrank_decompose.argtypes = [i64, i64, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, i64, vp]
        L.svdq_lowrank_decompose_noalloc.argtypes = [i64, i64, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp]
        L.svdq_quantize_weight.argtypes = [i32, i32, i64, i64, vp, f32, vp, vp, vp]
        L.awq_quantize_weight.argtypes = [i32, i64, i64, vp, vp, vp, vp, vp]
        L.svdq_w4a4_group_psums.argtypes = [i32, i32, i64, i64, i64, vp, vp, vp, vp]
        for f in ("svdq_quantize_act", "svdq_quantize_act_ws", "svdq_w4a4_gemm", "svdq_w4a4_gemm_ws", "svdq_w4a4_gemm_qkv_norm_rope",
                  "svdq_w4a4_gemm_qkv_norm_rope_ws",
                  "svdq_w4a4_gemm_gelu_quant", "awq_w4a16_gemv", "svdq_quantize_act_awq_gemv",
                  "svdq_w4a4_group_psums", "svdq_calibrate_smooth",
                  "svdq_lowrank_decompose", "svdq_lowrank_decompose_noalloc", "svdq_quantize_weight",
                  "awq_quantize_weight"):
            getattr(L, f).restype = i32
        L.svdq_last_error.restype = ctypes.c_char_p
        L.svdq_abi_version.restype = i32
        L.svdq_test_set_arch_override.argtypes = [ctypes.c_char_p]
        L.svdq_test_set_arch_override.restype = None
        L.svdq_test_set_no_ksplit.argtypes = [i32]
        L.svdq_test_set_no_ksplit.restype = None
        _lib = L
    return _lib


def _check(status: int) -> None:
    if status != 0:
        raise SvdqError(status, lib().svdq_last_error().decode())


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


_U8, _BF16, _F16, _F32, _I32 = torch.uint8, torch.bfloat16, torch.float16, torch.float32, torch.int32


def _scale_dtype(precision):
    return _F16 if precision == SVDQ_INT4 else _U8


class _Args:
    """Checks the tensors of one call before any pointer reaches the library: each
    is a torch.Tensor of the documented dtype and shape, contiguous, and every
    tensor lives on one GPU.  Shapes are checked first and the device last, so a
    call with host tensors fails here whatever else is wrong.  Raises ValueError."""

    def __init__(self, fn):
        self.fn, self.items = fn, []

    def req(self, name, t, dtype, shape, optional=False):
        if t is None:
            if not optional:
                raise ValueError(f"{self.fn}: {name} is required")
            return self
        if not isinstance(t, torch.Tensor):
            raise ValueError(f"{self.fn}: {name} must be a torch.Tensor, got {type(t).__name__}")
        if t.dtype != dtype:
            raise ValueError(f"{self.fn}: {name} must be {dtype}, got {t.dtype}")
        if tuple(t.shape) != tuple(int(v) for v in shape):
            raise ValueError(f"{self.fn}: {name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
        if not t.is_contiguous():
            raise ValueError(f"{self.fn}: {name} must be contiguous")
        self.items.append((name, t))
        return self

    def done(self):
        dev = None
        for name, t in self.items:
            if t.device.type != "cuda":
                raise ValueError(f"{self.fn}: {name} is on {t.device}, not on a GPU")
            if dev is None:
                dev = t.device
            elif t.device != dev:
                raise ValueError(f"{self.fn}: {name} is on {t.device}, the other tensors on {dev}")


def _dims(fn, t, name, nd):
    if not isinstance(t, torch.Tensor) or t.dim() != nd:
        raise ValueError(f"{fn}: {name} must be a {nd}-D torch.Tensor")
    return tuple(t.shape)


def quantize_act(precision: int, x, smooth=None, l1t=None, act_global_scale: float = 1.0,
                 out=None, stream=None, workspace=None):
    """svdq_quantize_act, or svdq_quantize_act_ws when `workspace` (see gemm_workspace;
    the same one may serve the GEMMs of the stream) is given.  x: bf16 [M, K]; smooth:
    bf16 [K] or None; l1t: bf16 [r, K] or None.  Returns (codes u8 [M, K/2], scales,
    xl1 fp32 [M, r] or None); `out` may supply that triple preallocated."""
    M, K = _dims("quantize_act", x, "x", 2)
    G = GROUP.get(precision, 64)
    r = 0 if l1t is None else _dims("quantize_act", l1t, "l1t", 2)[0]
    if out is None:
        codes = torch.empty((M, K // 2), dtype=_U8, device=x.device)
        scales = torch.empty((M, K // G), dtype=_scale_dtype(precision), device=x.device)
        xl1 = torch.empty((M, r), dtype=_F32, device=x.device) if r else None
    else:
        codes, scales, xl1 = out
    (_Args("quantize_act").req("x", x, _BF16, (M, K)).req("smooth", smooth, _BF16, (K,), True)
     .req("l1t", l1t, _BF16, (r, K), True).req("codes", codes, _U8, (M, K // 2))
     .req("scales", scales, _scale_dtype(precision), (M, K // G)).req("xl1", xl1, _F32, (M, r), r == 0)
     .req("workspace", workspace, _U8, (GEMM_WORK_BYTES,), True).done())
    args = (precision, G, r, M, K, _ptr(x), _ptr(smooth), _ptr(l1t), float(act_global_scale), _ptr(codes),
            _ptr(scales), _ptr(xl1))
    if workspace is None:
        _check(lib().svdq_quantize_act(*args, _stream(stream)))
    else:
        _check(lib().svdq_quantize_act_ws(*args, _ptr(workspace), GEMM_WORK_BYTES, _stream(stream)))
    return codes, scales, xl1


def _gemm_args(fn, precision, act_codes, act_scales, w_codes, w_scales, xl1, l2t, bias, N=None):
    M, Kh = _dims(fn, act_codes, "act_codes", 2)
    K = 2 * Kh
    if N is None:
        N = _dims(fn, w_codes, "w_codes", 2)[0]
    G = GROUP.get(precision, 64)
    r = 0 if l2t is None else _dims(fn, l2t, "l2t", 2)[1]
    a = (_Args(fn).req("act_codes", act_codes, _U8, (M, K // 2))
         .req("act_scales", act_scales, _scale_dtype(precision), (M, K // G))
         .req("w_codes", w_codes, _U8, (N, K // 2)).req("w_scales", w_scales, _scale_dtype(precision), (N, K // G))
         .req("xl1", xl1, _F32, (M, r), r == 0).req("l2t", l2t, _BF16, (N, r), True)
         .req("bias", bias, _BF16, (N,), True))
    if r == 0 and xl1 is not None:
        raise ValueError(f"{fn}: xl1 is given but l2t is not")
    return a, M, N, K, G, r


def gemm_workspace(device=None):
    """A zero-filled workspace for w4a4_gemm(..., workspace=): u8 [GEMM_WORK_BYTES] on
    `device`.  One per stream that may run GEMMs at the same time as another."""
    return torch.zeros((GEMM_WORK_BYTES,), dtype=_U8, device=device if device is not None else "cuda")


def w4a4_gemm(precision: int, act_codes, act_scales, w_codes, w_scales, xl1=None, l2t=None,
              bias=None, act_global_scale: float = 1.0, w_global_scale: float = 1.0, out=None,
              stream=None, workspace=None):
    """svdq_w4a4_gemm, or svdq_w4a4_gemm_ws when `workspace` (see gemm_workspace) is
    given.  Returns Y bf16 [M, N]."""
    a, M, N, K, G, r = _gemm_args("w4a4_gemm", precision, act_codes, act_scales, w_codes, w_scales, xl1, l2t, bias)
    y = out if out is not None else torch.empty((M, N), dtype=_BF16, device=act_codes.device)
    a.req("y", y, _BF16, (M, N)).req("workspace", workspace, _U8, (GEMM_WORK_BYTES,), True).done()
    args = (precision, G, r, M, N, K, _ptr(act_codes), _ptr(act_scales), float(act_global_scale), _ptr(w_codes),
            _ptr(w_scales), float(w_global_scale), _ptr(xl1), _ptr(l2t), _ptr(bias), _ptr(y))
    if workspace is None:
        _check(lib().svdq_w4a4_gemm(*args, _stream(stream)))
    else:
        _check(lib().svdq_w4a4_gemm_ws(*args, _ptr(workspace), GEMM_WORK_BYTES, _stream(stream)))
    return y


def w4a4_gemm_qkv_norm_rope(precision: int, act_codes, act_scales, w_codes, w_scales, xl1, l2t, bias,
                            heads: int, head_dim: int, norm_q, norm_k, eps: float, rope=None,
                            act_global_scale: float = 1.0, w_global_scale: float = 1.0, out=None,
                            stream=None, workspace=None):
    """svdq_w4a4_gemm_qkv_norm_rope (svdq_w4a4_gemm_qkv_norm_rope_ws when `workspace`, see
    gemm_workspace, is given): the fused attention projection.  w_codes holds the Q, K
    and V weights concatenated along N (= 3 * heads * head_dim); rope is fp32
    [S, head_dim/2, 2] (cos, sin) or None.  Returns Y bf16 [M, N]."""
    fn = "w4a4_gemm_qkv_norm_rope"
    N = 3 * int(heads) * int(head_dim)
    a, M, N, K, G, r = _gemm_args(fn, precision, act_codes, act_scales, w_codes, w_scales, xl1, l2t, bias, N)
    rope_rows = 0 if rope is None else _dims(fn, rope, "rope", 3)[0]
    y = out if out is not None else torch.empty((M, N), dtype=_BF16, device=act_codes.device)
    (a.req("norm_q", norm_q, _BF16, (head_dim,)).req("norm_k", norm_k, _BF16, (head_dim,))
     .req("rope", rope, _F32, (rope_rows, head_dim // 2, 2), True).req("y", y, _BF16, (M, N))
     .req("workspace", workspace, _U8, (GEMM_WORK_BYTES,), True).done())
    args = (precision, G, r, M, heads, head_dim, K, _ptr(act_codes), _ptr(act_scales), float(act_global_scale),
            _ptr(w_codes), _ptr(w_scales), float(w_global_scale), _ptr(xl1), _ptr(l2t), _ptr(bias), _ptr(norm_q),
            _ptr(norm_k), float(eps), _ptr(rope), rope_rows, _ptr(y))
    if workspace is None:
        _check(lib().svdq_w4a4_gemm_qkv_norm_rope(*args, _stream(stream)))
    else:
        _check(lib().svdq_w4a4_gemm_qkv_norm_rope_ws(*args, _ptr(workspace), GEMM_WORK_BYTES, _stream(stream)))
    return y


def w4a4_gemm_gelu_quant(act_codes, act_scales, w_codes, w_scales, xl1, l2t, bias, smooth_out=None,
                         l1t_out=None, out=None, stream=None, precision: int = SVDQ_INT4,
                         act_global_scale: float = 1.0, w_global_scale: float = 1.0,
                         out_global_scale: float = 1.0):
    """svdq_w4a4_gemm_gelu_quant: the MLP up-projection with GELU and the down
    projection's quantization fused (int4, or nvfp4 with the global scales of
    the up projection and out_global_scale for the quantization of h).
    Returns (codes u8 [M, N/2], scales [M, N/G] (fp16 for int4, E4M3 u8 for
    nvfp4), xl1 fp32 [M, r_out] or None); `out` may supply that triple
    preallocated."""
    fn = "w4a4_gemm_gelu_quant"
    a, M, N, K, G, r = _gemm_args(fn, precision, act_codes, act_scales, w_codes, w_scales, xl1, l2t, bias)
    ro = 0 if l1t_out is None else _dims(fn, l1t_out, "l1t_out", 2)[0]
    sdt = _scale_dtype(precision)
    if out is None:
        dev = act_codes.device
        out = (torch.empty((M, N // 2), dtype=_U8, device=dev), torch.empty((M, N // G), dtype=sdt, device=dev),
               torch.empty((M, ro), dtype=_F32, device=dev) if ro else None)
    codes, scales, xo = out
    (a.req("smooth_out", smooth_out, _BF16, (N,), True).req("l1t_out", l1t_out, _BF16, (ro, N), True)
     .req("codes_out", codes, _U8, (M, N // 2)).req("scales_out", scales, sdt, (M, N // G))
     .req("xl1_out", xo, _F32, (M, ro), ro == 0).done())
    _check(lib().svdq_w4a4_gemm_gelu_quant(
        precision, G, r, M, N, K, _ptr(act_codes), _ptr(act_scales), float(act_global_scale), _ptr(w_codes),
        _ptr(w_scales), float(w_global_scale), _ptr(xl1), _ptr(l2t), _ptr(bias), _ptr(smooth_out),
        _ptr(l1t_out), ro, float(out_global_scale), _ptr(codes), _ptr(scales), _ptr(xo), _stream(stream)))
    return codes, scales, xo


def calibrate_smooth(x_cal, w, out=None, stream=None):
    """svdq_calibrate_smooth: lambda bf16 [K] from calibration activations and the dense weight."""
    Mc, K = _dims("calibrate_smooth", x_cal, "x_cal", 2)
    N = _dims("calibrate_smooth", w, "w", 2)[0]
    lam = out if out is not None else torch.empty(K, dtype=_BF16, device=w.device)
    (_Args("calibrate_smooth").req("x_cal", x_cal, _BF16, (Mc, K)).req("w", w, _BF16, (N, K))
     .req("smooth_out", lam, _BF16, (K,)).done())
    _check(lib().svdq_calibrate_smooth(Mc, N, K, _ptr(x_cal), _ptr(w), _ptr(lam), _stream(stream)))
    return lam


def lowrank_decompose(w, smooth, omega, rank: int, iters: int = 4, stream=None):
    """svdq_lowrank_decompose: returns (l1t bf16 [rank, K], l2t bf16 [N, rank], residual fp32 [N, K]).
    omega: fp32 [K, rank + oversample] test matrix."""
    fn = "lowrank_decompose"
    N, K = _dims(fn, w, "w", 2)
    p = _dims(fn, omega, "omega", 2)[1]
    _Args(fn).req("w", w, _BF16, (N, K)).req("smooth", smooth, _BF16, (K,), True).req("omega", omega, _F32, (K, p)).done()
    nbytes = lib().svdq_lowrank_workspace_bytes(N, K, rank, p - rank)
    if nbytes < 0:
        raise SvdqError(2, f"unsupported decomposition sizes N={N} K={K} rank={rank} p={p}")
    dev = w.device
    work = torch.empty(nbytes, dtype=_U8, device=dev)
    l1t = torch.empty((rank, K), dtype=_BF16, device=dev)
    l2t = torch.empty((N, rank), dtype=_BF16, device=dev)
    res = torch.empty((N, K), dtype=_F32, device=dev)
    _check(lib().svdq_lowrank_decompose(N, K, rank, p - rank, iters, _ptr(w), _ptr(smooth), _ptr(omega), _ptr(l1t),
                                        _ptr(l2t), _ptr(res), _ptr(work), nbytes, _stream(stream)))
    return l1t, l2t, res


def quantize_weight(precision: int, residual, w_global_scale: float = 1.0, out=None, stream=None):
    """svdq_quantize_weight: (codes u8 [N, K/2], scales) of an fp32 residual [N, K]."""
    N, K = _dims("quantize_weight", residual, "residual", 2)
    G = GROUP.get(precision, 64)
    if out is None:
        out = (torch.empty((N, K // 2), dtype=_U8, device=residual.device),
               torch.empty((N, K // G), dtype=_scale_dtype(precision), device=residual.device))
    (_Args("quantize_weight").req("residual", residual, _F32, (N, K)).req("codes", out[0], _U8, (N, K // 2))
     .req("scales", out[1], _scale_dtype(precision), (N, K // G)).done())
    _check(lib().svdq_quantize_weight(precision, G, N, K, _ptr(residual), float(w_global_scale), _ptr(out[0]),
                                      _ptr(out[1]), _stream(stream)))
    return out


def awq_quantize_weight(w, out=None, stream=None):
    """awq_quantize_weight: (codes u8 [N, K/2], scales fp16 [N, K/64], zeros fp16 [N, K/64])."""
    N, K = _dims("awq_quantize_weight", w, "w", 2)
    if out is None:
        dev = w.device
        out = (torch.empty((N, K // 2), dtype=_U8, device=dev), torch.empty((N, K // 64), dtype=_F16, device=dev),
               torch.empty((N, K // 64), dtype=_F16, device=dev))
    (_Args("awq_quantize_weight").req("w", w, _BF16, (N, K)).req("codes", out[0], _U8, (N, K // 2))
     .req("scales", out[1], _F16, (N, K // 64)).req("zeros", out[2], _F16, (N, K // 64)).done())
    _check(lib().awq_quantize_weight(64, N, K, _ptr(w), _ptr(out[0]), _ptr(out[1]), _ptr(out[2]), _stream(stream)))
    return out


def group_psums(precision: int, act_codes, w_codes, out=None, stream=None):
    """svdq_w4a4_group_psums (test support).  Returns [M, N, K/G] int32 (int4) or fp32 (nvfp4).
    Row slices of larger code tensors (contiguous, so a pointer offset) crop the product."""
    M, Kh = _dims("group_psums", act_codes, "act_codes", 2)
    K = 2 * Kh
    N = _dims("group_psums", w_codes, "w_codes", 2)[0]
    G = GROUP.get(precision, 64)
    pdt = _I32 if precision == SVDQ_INT4 else _F32
    if out is None:
        out = torch.empty((M, N, K // G), dtype=pdt, device=act_codes.device)
    (_Args("group_psums").req("act_codes", act_codes, _U8, (M, K // 2)).req("w_codes", w_codes, _U8, (N, K // 2))
     .req("psums", out, pdt, (M, N, K // G)).done())
    _check(lib().svdq_w4a4_group_psums(precision, G, M, N, K, _ptr(act_codes), _ptr(w_codes),
                                       _ptr(out), _stream(stream)))
    return out


def awq_gemv(x, w_codes, w_scales, w_zeros, bias=None, out=None, stream=None, group_size: int = 64):
    """awq_w4a16_gemv.  x bf16 [M, K]; returns Y bf16 [M, N]."""
    M, K = _dims("awq_gemv", x, "x", 2)
    N = _dims("awq_gemv", w_codes, "w_codes", 2)[0]
    G = int(group_size) if group_size else 64
    y = out if out is not None else torch.empty((M, N), dtype=_BF16, device=x.device)
    (_Args("awq_gemv").req("x", x, _BF16, (M, K)).req("w_codes", w_codes, _U8, (N, K // 2))
     .req("w_scales", w_scales, _F16, (N, K // G)).req("w_zeros", w_zeros, _F16, (N, K // G))
     .req("bias", bias, _BF16, (N,), True).req("y", y, _BF16, (M, N)).done())
    _check(lib().awq_w4a16_gemv(group_size, M, N, K, _ptr(x), _ptr(w_codes), _ptr(w_scales),
                                _ptr(w_zeros), _ptr(bias), _ptr(y), _stream(stream)))
    return y


def quantize_act_awq_gemv(precision: int, x, smooth, l1t, act_global_scale: float, awq_x, w_codes, w_scales,
                          w_zeros, bias=None, out=None, awq_out=None, stream=None):
    """svdq_quantize_act_awq_gemv: quantize_act(precision, x, smooth, l1t, act_global_scale)
    and awq_gemv(awq_x, w_codes, w_scales, w_zeros, bias) in one launch where the shapes
    allow it.  Returns ((codes, scales, xl1), y); `out` / `awq_out` may supply the
    quantizer's triple and the AWQ output preallocated."""
    M, K = _dims("quantize_act_awq_gemv", x, "x", 2)
    G = GROUP.get(precision, 64)
    r = 0 if l1t is None else _dims("quantize_act_awq_gemv", l1t, "l1t", 2)[0]
    aM, aK = _dims("quantize_act_awq_gemv", awq_x, "awq_x", 2)
    aN = _dims("quantize_act_awq_gemv", w_codes, "w_codes", 2)[0]
    if out is None:
        codes = torch.empty((M, K // 2), dtype=_U8, device=x.device)
        scales = torch.empty((M, K // G), dtype=_scale_dtype(precision), device=x.device)
        xl1 = torch.empty((M, r), dtype=_F32, device=x.device) if r else None
    else:
        codes, scales, xl1 = out
    y = awq_out if awq_out is not None else torch.empty((aM, aN), dtype=_BF16, device=awq_x.device)
    (_Args("quantize_act_awq_gemv").req("x", x, _BF16, (M, K)).req("smooth", smooth, _BF16, (K,), True)
     .req("l1t", l1t, _BF16, (r, K), True).req("codes", codes, _U8, (M, K // 2))
     .req("scales", scales, _scale_dtype(precision), (M, K // G)).req("xl1", xl1, _F32, (M, r), r == 0)
     .req("awq_x", awq_x, _BF16, (aM, aK)).req("w_codes", w_codes, _U8, (aN, aK // 2))
     .req("w_scales", w_scales, _F16, (aN, aK // 64)).req("w_zeros", w_zeros, _F16, (aN, aK // 64))
     .req("bias", bias, _BF16, (aN,), True).req("y", y, _BF16, (aM, aN)).done())
    _check(lib().svdq_quantize_act_awq_gemv(precision, G, r, M, K, _ptr(x), _ptr(smooth), _ptr(l1t),
                                            float(act_global_scale), _ptr(codes), _ptr(scales), _ptr(xl1), 64,
                                            aM, aN, aK, _ptr(awq_x), _ptr(w_codes), _ptr(w_scales),
                                            _ptr(w_zeros), _ptr(bias), _ptr(y), _stream(stream)))
    return (codes, scales, xl1), y


def svdq_linear(precision: int, x, smooth, l1t, w_codes, w_scales, l2t, bias,
                act_global_scale: float = 1.0, w_global_scale: float = 1.0, stream=None):
    """The whole SVDQuant linear: quantize (+ X.L1) then the 4-bit GEMM (+ low-rank up, bias)."""
    codes, scales, xl1 = quantize_act(precision, x, smooth, l1t, act_global_scale, stream=stream)
    return w4a4_gemm(precision, codes, scales, w_codes, w_scales, xl1, l2t, bias,
                     act_global_scale, w_global_scale, stream=stream)


def abi_version() -> int:
    return lib().svdq_abi_version()


def set_no_ksplit(on: bool):
    """Test hook: force the int4 GEMM's one-copy kernel instance on small grids (False restores)."""
    lib().svdq_test_set_no_ksplit(1 if on else 0)


def set_arch_override(arch):
    """Test hook: make the architecture check see `arch` (None restores the device's)."""
    lib().svdq_test_set_arch_override(None if arch is None else arch.encode())
