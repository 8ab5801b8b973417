"""CPU oracle for the SVDQuant W4A4 linear and the AWQ W4A16 linear.

TEST INFRASTRUCTURE ONLY.  Only tests/, the smoke check in __graft_entry__ and
the cpu_baseline leg of bench.py may import this module.  The product path
(the HIP library and its Python binding) never imports it.

Every function here is a thin numpy <-> ctypes marshalling layer over
svdq_oracle.cpp; the arithmetic, and its citations of the pages, live there.
Arrays are numpy: bf16 and fp16 values travel as their uint16 bit patterns,
E4M3 scales as uint8, 4-bit codes as packed uint8 [rows, K/2].
"""
import ctypes
import os

import numpy as np

from . import build as _build

_LIB = None

INT4, NVFP4 = 0, 1


def _lib():
    global _LIB
    if _LIB is None:
        # SVDQ_ORACLE_LIB: another build of svdq_oracle.cpp (the sanitizer
        # test loads an ASan/UBSan build this way)
        path = os.environ.get("SVDQ_ORACLE_LIB")
        if not path:
            path = _build.LIB
            if not os.path.exists(path):
                _build.build()
        _LIB = ctypes.CDLL(path)
    return _LIB


def _p(a):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be contiguous"
    return a.ctypes.data_as(ctypes.c_void_p)


def _i64(v):
    return ctypes.c_int64(int(v))


# ---- converters -------------------------------------------------------------
def _vec(name, arr, out_dtype):
    arr = np.ascontiguousarray(arr)
    out = np.empty(arr.shape, dtype=out_dtype)
    getattr(_lib(), name)(_p(arr), _p(out), _i64(arr.size))
    return out


def f32_to_f16_sat(x):
    return _vec("orc_vec_f32_to_f16_sat", np.asarray(x, np.float32), np.uint16)


def f32_to_bf16(x):
    return _vec("orc_vec_f32_to_bf16", np.asarray(x, np.float32), np.uint16)


def f32_to_e4m3_sat(x):
    return _vec("orc_vec_f32_to_e4m3_sat", np.asarray(x, np.float32), np.uint8)


def f32_to_e2m1_sat(x):
    return _vec("orc_vec_f32_to_e2m1_sat", np.asarray(x, np.float32), np.uint8)


def f16_to_f32(h):
    return _vec("orc_vec_f16_to_f32", np.asarray(h, np.uint16), np.float32)


def bf16_to_f32(h):
    return _vec("orc_vec_bf16_to_f32", np.asarray(h, np.uint16), np.float32)


def e4m3_to_f32(b):
    return _vec("orc_vec_e4m3_to_f32", np.asarray(b, np.uint8), np.float32)


def e2m1_to_f32(c):
    return _vec("orc_vec_e2m1_to_f32", np.asarray(c, np.uint8), np.float32)


# ---- the method ---------------------------------------------------------------
def quantize_act(prec, x, lam=None, alpha=1.0, nthreads=0):
    """Returns (codes u8 [M, K/2], scales) for bf16 bits x [M, K]."""
    x = np.ascontiguousarray(x, dtype=np.uint16)
    M, K = x.shape
    lam = None if lam is None else np.ascontiguousarray(lam, dtype=np.uint16)
    codes = np.zeros((M, K // 2), np.uint8)
    if prec == INT4:
        scales = np.zeros((M, K // 64), np.uint16)
        _lib().orc_quantize_act_int4(_i64(M), _i64(K), _p(x), _p(lam), _p(codes), _p(scales),
                                     ctypes.c_int(nthreads))
    else:
        scales = np.zeros((M, K // 16), np.uint8)
        _lib().orc_quantize_act_nvfp4(_i64(M), _i64(K), _p(x), _p(lam), ctypes.c_float(alpha),
                                      _p(codes), _p(scales), ctypes.c_int(nthreads))
    return codes, scales


def lowrank_down(x, l1t, nthreads=0):
    """XL1 fp32 [M, r] from bf16 bits x [M, K] and l1t = L1^T [r, K]."""
    x = np.ascontiguousarray(x, dtype=np.uint16)
    l1t = np.ascontiguousarray(l1t, dtype=np.uint16)
    M, K = x.shape
    r = l1t.shape[0]
    out = np.zeros((M, r), np.float32)
    if r:
        _lib().orc_lowrank_down(_i64(M), _i64(K), ctypes.c_int(r), _p(x), _p(l1t), _p(out),
                                ctypes.c_int(nthreads))
    return out


def group_psums(prec, a_codes, w_codes, nthreads=0):
    a_codes = np.ascontiguousarray(a_codes, dtype=np.uint8)
    w_codes = np.ascontiguousarray(w_codes, dtype=np.uint8)
    M, K = a_codes.shape[0], a_codes.shape[1] * 2
    N = w_codes.shape[0]
    G = 64 if prec == INT4 else 16
    out = np.zeros((M, N, K // G), np.int32 if prec == INT4 else np.float32)
    _lib().orc_group_psums(ctypes.c_int(prec), _i64(M), _i64(N), _i64(K), _p(a_codes),
                           _p(w_codes), _p(out), ctypes.c_int(nthreads))
    return out


def w4a4_linear(prec, a_codes, a_scales, w_codes, w_scales, xl1=None, l2t=None, bias=None,
                alpha_a=1.0, alpha_w=1.0, rows=None, cols=None, nthreads=0):
    """Returns (y float64, y_bf16 uint16): full [M, N], or at (rows[i], cols[i])."""
    a_codes = np.ascontiguousarray(a_codes, dtype=np.uint8)
    w_codes = np.ascontiguousarray(w_codes, dtype=np.uint8)
    a_scales = np.ascontiguousarray(a_scales)
    w_scales = np.ascontiguousarray(w_scales)
    M, K = a_codes.shape[0], a_codes.shape[1] * 2
    N = w_codes.shape[0]
    r = 0 if l2t is None else l2t.shape[1]
    if r:
        xl1 = np.ascontiguousarray(xl1, dtype=np.float32)
        l2t = np.ascontiguousarray(l2t, dtype=np.uint16)
        assert xl1.shape == (M, r) and l2t.shape == (N, r)
    bias = None if bias is None else np.ascontiguousarray(bias, dtype=np.uint16)
    if rows is None:
        count = -1
        y = np.zeros((M, N), np.float64)
        yb = np.zeros((M, N), np.uint16)
        ri = ci = None
    else:
        ri = np.ascontiguousarray(rows, dtype=np.int64)
        ci = np.ascontiguousarray(cols, dtype=np.int64)
        count = ri.size
        y = np.zeros(count, np.float64)
        yb = np.zeros(count, np.uint16)
    _lib().orc_w4a4_linear(ctypes.c_int(prec), ctypes.c_int(r), _i64(M), _i64(N), _i64(K),
                           _p(a_codes), _p(a_scales), ctypes.c_float(alpha_a),
                           _p(w_codes), _p(w_scales), ctypes.c_float(alpha_w),
                           _p(xl1 if r else None), _p(l2t if r else None), _p(bias),
                           _i64(count), _p(ri), _p(ci), _p(y), _p(yb), ctypes.c_int(nthreads))
    return y, yb


def awq_linear(x, w_codes, w_scales, w_zeros, bias=None, rows=None, cols=None, nthreads=0):
    x = np.ascontiguousarray(x, dtype=np.uint16)
    w_codes = np.ascontiguousarray(w_codes, dtype=np.uint8)
    w_scales = np.ascontiguousarray(w_scales, dtype=np.uint16)
    w_zeros = np.ascontiguousarray(w_zeros, dtype=np.uint16)
    bias = None if bias is None else np.ascontiguousarray(bias, dtype=np.uint16)
    M, K = x.shape
    N = w_codes.shape[0]
    if rows is None:
        count = -1
        y = np.zeros((M, N), np.float64)
        yb = np.zeros((M, N), np.uint16)
        ri = ci = None
    else:
        ri = np.ascontiguousarray(rows, dtype=np.int64)
        ci = np.ascontiguousarray(cols, dtype=np.int64)
        count = ri.size
        y = np.zeros(count, np.float64)
        yb = np.zeros(count, np.uint16)
    _lib().orc_awq_linear(_i64(M), _i64(N), _i64(K), _p(x), _p(w_codes), _p(w_scales),
                          _p(w_zeros), _p(bias), _i64(count), _p(ri), _p(ci), _p(y), _p(yb),
                          ctypes.c_int(nthreads))
    return y, yb


def qkv_norm_rope(y, row_ids, heads, head_dim, norm_q, norm_k, eps, rope=None):
    """Q/K RMSNorm + rotary epilogue on the projection y float64 [rows, 3*heads*D] of
    tokens row_ids; returns (y float64, y_bf16 uint16) of the same shape."""
    y = np.ascontiguousarray(y, dtype=np.float64)
    rows = y.shape[0]
    assert y.shape[1] == 3 * heads * head_dim
    rid = np.ascontiguousarray(row_ids if row_ids is not None else np.arange(rows), dtype=np.int64)
    nq = np.ascontiguousarray(norm_q, dtype=np.uint16)
    nk = np.ascontiguousarray(norm_k, dtype=np.uint16)
    assert nq.shape == (head_dim,) and nk.shape == (head_dim,)
    rope_rows = 0
    if rope is not None:
        rope = np.ascontiguousarray(rope, dtype=np.float32)
        assert rope.shape[1:] == (head_dim // 2, 2)
        rope_rows = rope.shape[0]
    out = np.zeros_like(y)
    outb = np.zeros(y.shape, np.uint16)
    _lib().orc_qkv_norm_rope(_i64(rows), ctypes.c_int(heads), ctypes.c_int(head_dim), _p(y), _p(rid),
                             _p(nq), _p(nk), ctypes.c_double(eps), _p(rope), _i64(rope_rows),
                             _p(out), _p(outb))
    return out, outb


def w4a4_linear_qkv(prec, a_codes, a_scales, w_codes, w_scales, xl1, l2t, bias, heads, head_dim,
                    norm_q, norm_k, eps, rope=None, alpha_a=1.0, alpha_w=1.0, rows=None, nthreads=0):
    """The fused attention projection: w4a4_linear over whole rows (all of them, or the
    token rows `rows`), then qkv_norm_rope.  Returns (y float64, y_bf16) [rows, N]."""
    M, N = a_codes.shape[0], w_codes.shape[0]
    rid = np.arange(M, dtype=np.int64) if rows is None else np.asarray(rows, np.int64)
    ri = np.repeat(rid, N)
    ci = np.tile(np.arange(N, dtype=np.int64), rid.size)
    y, _ = w4a4_linear(prec, a_codes, a_scales, w_codes, w_scales, xl1, l2t, bias, alpha_a=alpha_a,
                       alpha_w=alpha_w, rows=ri, cols=ci, nthreads=nthreads)
    return qkv_norm_rope(y.reshape(rid.size, N), rid, heads, head_dim, norm_q, norm_k, eps, rope)


def gelu(y):
    """GELU (erf form) of float64 y in double; returns (h float64, h_bf16 uint16)."""
    y = np.ascontiguousarray(y, dtype=np.float64)
    h = np.zeros_like(y)
    hb = np.zeros(y.shape, np.uint16)
    _lib().orc_gelu(_i64(y.size), _p(y), _p(h), _p(hb))
    return h, hb


def smooth(x, lam=None):
    """The smoothed fp32 activation xh = fl32(x * fl32(1/lambda)) the quantizer rounds."""
    x = np.ascontiguousarray(x, dtype=np.uint16)
    M, K = x.shape
    lam = None if lam is None else np.ascontiguousarray(lam, dtype=np.uint16)
    out = np.zeros((M, K), np.float32)
    _lib().orc_smooth(_i64(M), _i64(K), _p(x), _p(lam), _p(out))
    return out


def mlp_up_gelu_quant(a_codes, a_scales, w_codes, w_scales, xl1, l2t, bias, lam_down, l1t_down,
                      rows=None, nthreads=0, prec=INT4, alpha_a=1.0, alpha_w=1.0, alpha_out=1.0):
    """The fused MLP up-projection: the up linear y (precision prec, global scales
    alpha_a, alpha_w for nvfp4) over whole rows (all of them, or the token rows
    `rows`), h = bf16(GELU(y)), then the down-projection's activation quantization of h
    in the same precision (smoothing lam_down; nvfp4 global scale alpha_out) and its
    low-rank input XL1 = h . L1_down.  Returns dict(y, h_bf16, codes, scales, xl1, xh)."""
    M, N = a_codes.shape[0], w_codes.shape[0]
    rid = np.arange(M, dtype=np.int64) if rows is None else np.asarray(rows, np.int64)
    y, _ = w4a4_linear(prec, a_codes, a_scales, w_codes, w_scales, xl1, l2t, bias, alpha_a=alpha_a,
                       alpha_w=alpha_w, rows=np.repeat(rid, N), cols=np.tile(np.arange(N, dtype=np.int64), rid.size),
                       nthreads=nthreads)
    y = y.reshape(rid.size, N)
    _, hb = gelu(y)
    codes, scales = quantize_act(prec, hb, lam_down, alpha=alpha_out, nthreads=nthreads)
    xl1_down = lowrank_down(hb, l1t_down, nthreads=nthreads)
    return dict(y=y, h_bf16=hb, codes=codes, scales=scales, xl1=xl1_down, xh=smooth(hb, lam_down))


def f64_to_bf16(x):
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.zeros(x.shape, np.uint16)
    _lib().orc_vec_f64_to_bf16(_p(x), _p(out), _i64(x.size))
    return out


def calibrate_smooth(x_cal, w):
    """Smoothing factor lambda bf16 [K] from a calibration batch x_cal bf16 [Mc, K] and the
    dense weight w bf16 [N, K]: bf16(sqrt(fl32(max|x_k| / max|w_k|))), 1 if either is 0."""
    x_cal = np.ascontiguousarray(x_cal, dtype=np.uint16)
    w = np.ascontiguousarray(w, dtype=np.uint16)
    lam = np.zeros(w.shape[1], np.uint16)
    _lib().orc_calibrate_smooth(_i64(x_cal.shape[0]), _i64(w.shape[0]), _i64(w.shape[1]), _p(x_cal), _p(w),
                                _p(lam))
    return lam


def lowrank_decompose(w, lam, rank):
    """The rank-r branch of SVDQuant from the dense weight w bf16 [N, K] and lambda bf16 [K].
    Definition (double): W_hat = W diag(lambda) (the smoothed weight, so that
    (X / lambda) W_hat^T = X W^T); W_hat = U S V^T (numpy SVD); the best rank-r
    approximation (Eckart-Young) is U_r S_r V_r^T, split evenly between the factors and
    moved back to raw X for the layer:  L1 = diag(1/lambda) V_r S_r^(1/2) [K, r],
    L2 = S_r^(1/2) U_r^T [r, N].  Returns dict(l1t = bf16(L1^T) [r, K], l2t = bf16(L2^T)
    [N, r], lowrank = U_r S_r V_r^T, residual = W_hat - (diag(lambda) L1b L2b)^T, the part
    the 4-bit weight must carry given the stored bf16 factors L1b, L2b, w_hat, sigma)."""
    wf = bf16_to_f32(np.ascontiguousarray(w, dtype=np.uint16)).astype(np.float64)
    lamf = bf16_to_f32(np.ascontiguousarray(lam, dtype=np.uint16)).astype(np.float64)
    w_hat = wf * lamf[None, :]
    U, S, Vt = np.linalg.svd(w_hat, full_matrices=False)
    Ur, Sr, Vr = U[:, :rank], S[:rank], Vt[:rank, :].T
    sq = np.sqrt(Sr)
    l1 = (Vr * sq[None, :]) / lamf[:, None]          # [K, r]
    l2 = (Ur * sq[None, :]).T                         # [r, N]
    l1t = f64_to_bf16(l1.T)
    l2t = f64_to_bf16(l2.T)
    l1b = bf16_to_f32(l1t).astype(np.float64).T       # [K, r]
    l2b = bf16_to_f32(l2t).astype(np.float64).T       # [r, N]
    lowrank_b = ((lamf[:, None] * l1b) @ l2b).T       # [N, K]
    return dict(l1t=l1t, l2t=l2t, lowrank=(Ur * Sr[None, :]) @ Vr.T, residual=w_hat - lowrank_b,
                w_hat=w_hat, sigma=S)


def quantize_weight(prec, r, alpha=1.0):
    """4-bit codes and scales of an fp32 residual r [N, K] (int4 group 64 / nvfp4 group 16)."""
    r = np.ascontiguousarray(r, dtype=np.float32)
    N, K = r.shape
    G = 64 if prec == INT4 else 16
    codes = np.zeros((N, K // 2), np.uint8)
    scales = np.zeros((N, K // G), np.uint16 if prec == INT4 else np.uint8)
    _lib().orc_quantize_weight(ctypes.c_int(prec), _i64(N), _i64(K), _p(r), ctypes.c_float(alpha), _p(codes),
                               _p(scales))
    return codes, scales


def awq_quantize_weight(w):
    """AWQ int4 weight-only quantization of w bf16 [N, K]: (codes u8 [N, K/2], scales fp16
    [N, K/64], zero-points fp16 [N, K/64]), min-max over a range containing 0."""
    w = np.ascontiguousarray(w, dtype=np.uint16)
    N, K = w.shape
    codes = np.zeros((N, K // 2), np.uint8)
    scales = np.zeros((N, K // 64), np.uint16)
    zeros = np.zeros((N, K // 64), np.uint16)
    _lib().orc_awq_quantize_weight(_i64(N), _i64(K), _p(w), _p(codes), _p(scales), _p(zeros))
    return codes, scales, zeros
