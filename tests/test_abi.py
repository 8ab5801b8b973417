"""The C ABI on a host without a GPU: libsvdq.so loads, exports every function
that include/svdq.h declares, and rejects bad arguments and non-gfx950
devices before anything is launched (no compute call is made here: every
call below fails validation or the architecture check first)."""
import ctypes
import os
import re

import pytest

import bit_w4a4_quantized_smooth_amd as sq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "svdq.h")

OK, INVALID, UNSUPPORTED, ALIGN, DEVICE = 0, 1, 2, 3, 4
A = 1 << 20  # a fake, 16-byte aligned "device address"; never dereferenced


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(svdq_\w+|awq_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    return sq.lib()


@pytest.fixture(autouse=True)
def gfx942(L):
    # every call that gets past validation meets a non-gfx950 architecture
    L.svdq_test_set_arch_override(b"gfx942")
    yield
    L.svdq_test_set_arch_override(None)


def test_exports_every_declared_symbol(L):
    names = declared_functions()
    assert {"svdq_quantize_act", "svdq_w4a4_gemm", "awq_w4a16_gemv", "svdq_w4a4_group_psums",
            "svdq_last_error", "svdq_abi_version", "svdq_test_set_arch_override"} <= set(names)
    for n in names:
        assert hasattr(L, n), n
    assert set(sq.EXPORTS) == set(names)
    assert L.svdq_abi_version() == 1


def q(L, prec=0, G=64, r=16, M=256, K=512, x=A, smooth=A, l1t=A, alpha=1.0, codes=2 * A,
      scales=3 * A, xl1=4 * A):
    return L.svdq_quantize_act(prec, G, r, M, K, x, smooth, l1t, alpha, codes, scales, xl1, None)


def gemm(L, prec=0, G=64, r=16, M=256, N=512, K=512, ac=A, as_=2 * A, aa=1.0, wc=3 * A, ws=4 * A,
         aw=1.0, xl1=5 * A, l2t=6 * A, bias=7 * A, y=8 * A):
    return L.svdq_w4a4_gemm(prec, G, r, M, N, K, ac, as_, aa, wc, ws, aw, xl1, l2t, bias, y, None)


def awq(L, G=64, M=2, N=512, K=512, x=A, wc=2 * A, ws=3 * A, wz=4 * A, bias=5 * A, y=6 * A):
    return L.awq_w4a16_gemv(G, M, N, K, x, wc, ws, wz, bias, y, None)


def test_valid_arguments_reach_the_arch_check(L):
    assert q(L) == UNSUPPORTED
    assert b"gfx942" in L.svdq_last_error()
    assert q(L, prec=1, G=16, alpha=0.01) == UNSUPPORTED
    assert gemm(L) == UNSUPPORTED
    assert gemm(L, prec=1, G=16) == UNSUPPORTED
    assert awq(L) == UNSUPPORTED
    assert L.svdq_w4a4_group_psums(0, 64, 256, 512, 512, A, 2 * A, 3 * A, None) == UNSUPPORTED


def test_precision_group_table(L):
    # the supported (method, precision, group) triples only
    assert q(L, prec=0, G=16) == UNSUPPORTED
    assert q(L, prec=1, G=64) == UNSUPPORTED
    assert q(L, prec=2, G=64) == UNSUPPORTED
    assert gemm(L, prec=0, G=32) == UNSUPPORTED
    assert awq(L, G=16) == UNSUPPORTED
    assert awq(L, G=128) == UNSUPPORTED


def test_rank_and_shape_limits(L):
    for r in (8, 24, 144, -16):
        assert q(L, r=r) == UNSUPPORTED
    assert q(L, K=96) == UNSUPPORTED          # not a multiple of 64
    assert q(L, M=-1) == INVALID
    assert q(L, K=0) == INVALID
    assert gemm(L, N=500) == UNSUPPORTED      # N % 128
    assert gemm(L, N=0) == INVALID
    assert awq(L, M=65) == UNSUPPORTED
    assert awq(L, N=96) == UNSUPPORTED
    # x stays below 2 GiB (32-bit buffer ranges): M*K < 2^30
    assert q(L, M=1 << 15, K=1 << 15) == UNSUPPORTED and b"2^30" in L.svdq_last_error()
    q(L, M=(1 << 15) - 1, K=1 << 15)
    assert b"2^30" not in L.svdq_last_error()
    assert awq(L, M=64, N=64, K=1 << 24) == UNSUPPORTED and b"2^30" in L.svdq_last_error()
    awq(L, M=63, N=64, K=1 << 24)
    assert b"2^30" not in L.svdq_last_error()


def test_required_pointers(L):
    assert q(L, x=None) == INVALID
    assert q(L, codes=None) == INVALID
    assert q(L, r=16, l1t=None) == INVALID
    assert q(L, r=0, l1t=A, xl1=None) == INVALID
    assert q(L, r=16, xl1=None) == INVALID
    assert q(L, r=0, l1t=None, xl1=None) == UNSUPPORTED  # valid: reaches the arch check
    assert q(L, smooth=None) == UNSUPPORTED              # smoothing is optional
    assert gemm(L, y=None) == INVALID
    assert gemm(L, r=16, l2t=None) == INVALID
    assert gemm(L, bias=None) == UNSUPPORTED             # bias is optional
    assert awq(L, wz=None) == INVALID
    assert q(L, prec=1, G=16, alpha=0.0) == INVALID
    assert q(L, prec=1, G=16, alpha=float("inf")) == INVALID


def test_alignment(L):
    assert q(L, x=A + 8) == ALIGN
    assert gemm(L, y=8 * A + 2) == ALIGN
    assert awq(L, ws=3 * A + 4) == ALIGN


def test_overlapping_outputs(L):
    assert q(L, codes=A) == INVALID  # codes alias x
    assert gemm(L, y=A) == INVALID   # y aliases act_codes


def test_empty_call_is_valid(L):
    L.svdq_test_set_arch_override(b"gfx950")
    assert q(L, M=0) == OK
    assert gemm(L, M=0) == OK
    assert awq(L, M=0) == OK


def test_python_binding_raises_loudly(L):
    with pytest.raises(sq.SvdqError) as e:
        sq._check(q(L))
    assert e.value.status == UNSUPPORTED


def qkv(L, prec=0, G=64, r=16, M=256, H=24, D=128, K=512, ac=A, as_=2 * A, aa=1.0, wc=3 * A, ws=4 * A,
        aw=1.0, xl1=5 * A, l2t=6 * A, bias=7 * A, nq=9 * A, nk=10 * A, eps=1e-6, rope=11 * A, rope_rows=256,
        y=12 * A):
    return L.svdq_w4a4_gemm_qkv_norm_rope(prec, G, r, M, H, D, K, ac, as_, aa, wc, ws, aw, xl1, l2t, bias,
                                          nq, nk, eps, rope, rope_rows, y, None)


def test_qkv_entry_point_validation(L):
    assert qkv(L) == UNSUPPORTED                      # valid: reaches the arch check
    assert qkv(L, prec=1, G=16) == UNSUPPORTED
    assert qkv(L, rope=None, rope_rows=0) == UNSUPPORTED  # the rotary table is optional
    assert qkv(L, bias=None) == UNSUPPORTED
    assert qkv(L, D=96) == UNSUPPORTED                # head_dim 64 or 128
    assert qkv(L, D=64, H=1) == UNSUPPORTED           # N = 192 is not a multiple of 128
    assert qkv(L, D=64, H=2) == UNSUPPORTED           # N = 384: valid
    assert qkv(L, H=0) == INVALID
    assert qkv(L, eps=-1e-6) == INVALID
    assert qkv(L, eps=float("nan")) == INVALID
    assert qkv(L, rope_rows=0) == INVALID
    assert qkv(L, nq=None) == INVALID
    assert qkv(L, nk=None) == INVALID
    assert qkv(L, y=None) == INVALID
    assert qkv(L, rope=11 * A + 4) == ALIGN
    assert qkv(L, nk=10 * A + 2) == ALIGN
    assert qkv(L, y=11 * A) == INVALID                # y aliases the rotary table
    assert qkv(L, y=9 * A) == INVALID                 # y aliases norm_q
    L.svdq_test_set_arch_override(b"gfx950")
    assert qkv(L, M=0) == OK


def mlp(L, prec=0, G=64, r=16, M=256, N=512, K=512, ac=A, as_=2 * A, wc=3 * A, ws=4 * A, xl1=5 * A, l2t=6 * A,
        bias=7 * A, lam=9 * A, l1t=10 * A, ro=32, co=11 * A, so=12 * A, xo=13 * A, aa=1.0, aw=1.0, ao=1.0):
    return L.svdq_w4a4_gemm_gelu_quant(prec, G, r, M, N, K, ac, as_, aa, wc, ws, aw, xl1, l2t, bias, lam, l1t,
                                       ro, ao, co, so, xo, None)


def test_mlp_entry_point_validation(L):
    assert mlp(L) == UNSUPPORTED                       # valid: reaches the arch check
    assert mlp(L, lam=None) == UNSUPPORTED             # smoothing is optional
    assert mlp(L, ro=0, l1t=None, xo=None) == UNSUPPORTED
    assert mlp(L, prec=1, G=16) == UNSUPPORTED         # nvfp4: valid, reaches the arch check
    assert mlp(L, prec=1, G=64) == UNSUPPORTED         # nvfp4 takes group 16
    assert mlp(L, prec=1, G=16, ao=0.0) == INVALID     # nvfp4: out_global_scale must be > 0
    assert mlp(L, prec=1, G=16, ao=float("inf")) == INVALID
    assert mlp(L, prec=1, G=16, ao=1e-39) == INVALID   # 6 * it would not be a normal float
    assert mlp(L, prec=1, G=16, aa=1e20, aw=1e20) == INVALID  # product of the up projection's scales overflows
    assert mlp(L, ao=0.0) == UNSUPPORTED               # int4 ignores the global scales
    assert mlp(L, ro=24) == UNSUPPORTED
    assert mlp(L, N=500) == UNSUPPORTED
    assert mlp(L, ro=32, l1t=None) == INVALID
    assert mlp(L, ro=32, xo=None) == INVALID
    assert mlp(L, co=None) == INVALID
    assert mlp(L, so=None) == INVALID
    assert mlp(L, co=11 * A + 8) == ALIGN
    assert mlp(L, co=A) == INVALID                     # codes_out aliases act_codes
    assert mlp(L, xo=12 * A) == INVALID                # xl1_out aliases scales_out
    L.svdq_test_set_arch_override(b"gfx950")
    assert mlp(L, M=0) == OK


def test_offline_entry_points_validation(L):
    assert L.svdq_calibrate_smooth(64, 128, 256, A, 2 * A, 3 * A, None) == UNSUPPORTED
    assert L.svdq_calibrate_smooth(64, 128, 255, A, 2 * A, 3 * A, None) == INVALID   # K even
    assert L.svdq_calibrate_smooth(64, 128, 256, A, 2 * A, A, None) == INVALID       # output aliases x
    assert L.svdq_lowrank_workspace_bytes(512, 256, 32, 16) > 0
    assert L.svdq_lowrank_workspace_bytes(512, 256, 32, 40) == -1                    # rank + oversample > 64
    ws = L.svdq_lowrank_workspace_bytes(512, 256, 32, 16)
    dec = lambda **k: L.svdq_lowrank_decompose(k.get("N", 512), k.get("K", 256), k.get("rank", 32), k.get("os", 16),
                                               k.get("it", 4), A, 2 * A, 3 * A, 4 * A, 5 * A, 8 * A, 16 * A,
                                               k.get("ws", ws), None)
    assert dec() == UNSUPPORTED
    assert dec(rank=24) == UNSUPPORTED
    assert dec(K=200) == INVALID
    assert dec(ws=ws - 1) == INVALID
    assert dec(it=-1) == INVALID
    assert L.svdq_quantize_weight(0, 64, 128, 256, A, 1.0, 2 * A, 3 * A, None) == UNSUPPORTED
    assert L.svdq_quantize_weight(1, 16, 128, 256, A, 0.0, 2 * A, 3 * A, None) == INVALID
    assert L.svdq_quantize_weight(0, 16, 128, 256, A, 1.0, 2 * A, 3 * A, None) == UNSUPPORTED
    assert L.awq_quantize_weight(64, 128, 256, A, 2 * A, 3 * A, 4 * A, None) == UNSUPPORTED
    assert L.awq_quantize_weight(32, 128, 256, A, 2 * A, 3 * A, 4 * A, None) == UNSUPPORTED
    assert L.awq_quantize_weight(64, 128, 256, A, A, 3 * A, 4 * A, None) == INVALID


def test_offset_and_k_limits(L):
    B = 1 << 36  # fake buffers far enough apart not to overlap at these sizes
    big = dict(ac=B, as_=2 * B, wc=3 * B, ws=4 * B, xl1=5 * B, l2t=6 * B, bias=7 * B, y=8 * B)
    # the GEMMs take K up to 32768, the largest K they are parity-tested at
    assert gemm(L, K=32768, **big) == UNSUPPORTED and b"gfx942" in L.svdq_last_error()
    assert gemm(L, K=32768 + 64, **big) == UNSUPPORTED and b"32768" in L.svdq_last_error()
    # xl1 [M, rank] fp32 and l2t [N, rank] bf16 are addressed with 32-bit byte offsets
    assert gemm(L, M=1 << 22, N=128, K=64, r=128, **big) == UNSUPPORTED and b"rank" in L.svdq_last_error()
    assert gemm(L, M=(1 << 22) - 1, N=128, K=64, r=128, **big) == UNSUPPORTED and b"gfx942" in L.svdq_last_error()
    assert gemm(L, M=64, N=1 << 23, K=64, r=128, **big) == UNSUPPORTED and b"rank" in L.svdq_last_error()
    bq = dict(x=B, smooth=2 * B, l1t=3 * B, codes=4 * B, scales=5 * B, xl1=6 * B)
    assert q(L, M=1 << 22, K=64, r=128, **bq) == UNSUPPORTED and b"rank" in L.svdq_last_error()
    assert q(L, M=(1 << 22) - 1, K=64, r=128, **bq) == UNSUPPORTED and b"gfx942" in L.svdq_last_error()
    assert mlp(L, M=1 << 22, N=128, K=64, r=0, ac=B, as_=2 * B, wc=3 * B, ws=4 * B, xl1=None, l2t=None, bias=7 * B,
               lam=9 * B, l1t=10 * B, ro=128, co=11 * B, so=12 * B, xo=13 * B) == UNSUPPORTED
    assert b"rank_out" in L.svdq_last_error()


def test_nvfp4_global_scale_product(L):
    # each scale is valid alone, but the factor fl32(alpha_a * alpha_w) the
    # epilogue applies overflows or underflows
    assert gemm(L, prec=1, G=16, aa=1e20, aw=1e20) == INVALID and b"normal" in L.svdq_last_error()
    assert gemm(L, prec=1, G=16, aa=1e-20, aw=1e-20) == INVALID
    assert gemm(L, prec=1, G=16, aa=1e-18, aw=1e-18) == UNSUPPORTED      # 1e-36 is normal: valid
    assert qkv(L, prec=1, G=16, aa=3e38, aw=2.0) == INVALID
    assert gemm(L, prec=0, G=64, aa=1e20, aw=1e20) == UNSUPPORTED        # int4 ignores them


def test_noalloc_decompose_limits(L):
    B = 1 << 40
    na = lambda N, K, r=32, os=16: L.svdq_lowrank_decompose_noalloc(N, K, r, os, 4, B, 2 * B, 3 * B, 4 * B, 5 * B,
                                                                    6 * B, None)
    assert na(1536, 768) == UNSUPPORTED and b"gfx942" in L.svdq_last_error()    # fits: reaches the arch check
    # a workspace above the fixed 16 MiB scratch is rejected, not run
    assert L.svdq_lowrank_workspace_bytes(1 << 17, 3072, 48, 16) > (16 << 20)
    assert na(1 << 17, 3072, 48, 16) == UNSUPPORTED and b"allocation-free limit" in L.svdq_last_error()
    assert na(1536, 768, r=24) == UNSUPPORTED                                   # the same rank rules
    assert L.svdq_lowrank_decompose_noalloc(1536, 768, 32, 16, 4, None, 2 * B, 3 * B, 4 * B, 5 * B, 6 * B,
                                            None) == INVALID


def gemm_ws(L, work=64 * A, work_bytes=sq.GEMM_WORK_BYTES, prec=0, G=64, M=256, y=8 * A, ac=A):
    return L.svdq_w4a4_gemm_ws(prec, G, 16, M, 512, 512, ac, 2 * A, 1.0, 3 * A, 4 * A, 1.0, 5 * A, 6 * A, 7 * A, y,
                               work, work_bytes, None)


def test_gemm_workspace_size_matches_the_header():
    text = open(HEADER).read()
    m = re.search(r"#define\s+SVDQ_GEMM_WORK_BYTES\s+\(\(int64_t\)\s*16\s*\*\s*1024\s*\*\s*1024\s*\+\s*4096\)", text)
    assert m, "SVDQ_GEMM_WORK_BYTES definition changed"
    assert sq.GEMM_WORK_BYTES == 16 * 1024 * 1024 + 4096


def test_gemm_workspace_validation(L):
    assert gemm_ws(L) == UNSUPPORTED                              # valid: reaches the arch check
    assert gemm_ws(L, work=None, work_bytes=0) == UNSUPPORTED     # no workspace: the plain GEMM
    assert gemm_ws(L, prec=1, G=16) == UNSUPPORTED                # nvfp4: the workspace is ignored
    assert gemm_ws(L, work=None, work_bytes=4096) == INVALID      # a size without a buffer
    assert gemm_ws(L, work_bytes=sq.GEMM_WORK_BYTES - 1) == INVALID and b"SVDQ_GEMM_WORK_BYTES" in L.svdq_last_error()
    assert gemm_ws(L, work=64 * A + 8) == ALIGN
    assert gemm_ws(L, work=8 * A - 4096) == INVALID               # overlaps y
    assert gemm_ws(L, work=A - 4096) == INVALID                   # overlaps act_codes
    assert gemm_ws(L, y=None) == INVALID                          # the plain GEMM's own checks still apply
    L.svdq_test_set_arch_override(b"gfx950")
    assert gemm_ws(L, M=0) == OK


def test_qkv_workspace_validation(L):
    def qkv_ws(work=64 * A, work_bytes=sq.GEMM_WORK_BYTES, y=8 * A):
        return L.svdq_w4a4_gemm_qkv_norm_rope_ws(0, 64, 16, 256, 2, 128, 512, A, 2 * A, 1.0, 3 * A, 4 * A, 1.0,
                                                 5 * A, 6 * A, 7 * A, 9 * A, 10 * A, 1e-6, 11 * A, 256, y,
                                                 work, work_bytes, None)
    assert qkv_ws() == UNSUPPORTED                                # valid: reaches the arch check
    assert qkv_ws(work=None, work_bytes=0) == UNSUPPORTED
    assert qkv_ws(work_bytes=4096) == INVALID
    assert qkv_ws(work=64 * A + 4) == ALIGN
    assert qkv_ws(work=10 * A - 4096) == INVALID                  # overlaps norm_k
    assert qkv_ws(work=8 * A - 4096) == INVALID                   # overlaps y


def test_quantize_workspace_validation(L):
    def qws(work=64 * A, work_bytes=sq.GEMM_WORK_BYTES, M=256, codes=2 * A, x=A):
        return L.svdq_quantize_act_ws(0, 64, 16, M, 512, x, None, 3 * A, 1.0, codes, 4 * A, 5 * A, work, work_bytes,
                                      None)
    assert qws() == UNSUPPORTED                                   # valid: reaches the arch check
    assert qws(work=None, work_bytes=0) == UNSUPPORTED            # no workspace: the plain quantizer
    assert qws(work=None, work_bytes=4096) == INVALID             # a size without a buffer
    assert qws(work_bytes=sq.GEMM_WORK_BYTES - 1) == INVALID and b"SVDQ_GEMM_WORK_BYTES" in L.svdq_last_error()
    assert qws(work=64 * A + 8) == ALIGN
    assert qws(work=A - 4096) == INVALID                          # overlaps x
    assert qws(work=2 * A - 4096) == INVALID                      # overlaps the codes
    assert qws(codes=None) == INVALID                             # the plain quantizer's own checks still apply
    L.svdq_test_set_arch_override(b"gfx950")
    assert qws(M=0) == OK


def test_quantize_awq_entry_validation(L):
    def qa(codes=2 * A, y=9 * A, awq_x=5 * A, aM=2, rank=16, l1t=3 * A, xl1=4 * A, M=256, ag=64):
        return L.svdq_quantize_act_awq_gemv(0, 64, rank, M, 512, A, None, l1t, 1.0, codes, 6 * A, xl1,
                                            ag, aM, 512, 512, awq_x, 7 * A, 8 * A, 10 * A, None, y, None)
    assert qa() == UNSUPPORTED                                    # valid: reaches the arch check
    assert qa(ag=128) == UNSUPPORTED and b"group 64" in L.svdq_last_error()   # the AWQ call's own checks
    assert qa(codes=None) == INVALID                              # the quantizer's own checks
    assert qa(y=A) == INVALID and b"AWQ output" in L.svdq_last_error()        # y over the quantizer's x
    assert qa(y=2 * A) == INVALID                                 # y over the codes
    assert qa(awq_x=2 * A) == INVALID and b"AWQ inputs" in L.svdq_last_error()  # codes over the AWQ x
    assert qa(M=0, aM=0) == OK                                    # both jobs empty: nothing enqueued
