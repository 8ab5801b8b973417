"""The allocation-free decomposition entry point (svdq_lowrank_decompose_noalloc),
called through the C ABI, against the allocating svdq_lowrank_decompose on the
same inputs: the two share every kernel and summation order, so the factors and
the residual must agree bit for bit.  Two calls in a row, the second smaller,
so the second runs on the scratch area the first left behind."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import bit_w4a4_quantized_smooth_amd as sq
from bit_w4a4_quantized_smooth_amd import synth

pytestmark = pytest.mark.gpu


def dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    return (t.view(dtype) if dtype is not None else t).cuda()


def b16(bits):
    return dev(np.asarray(bits, np.uint16).view(np.int16), torch.bfloat16)


def noalloc(w, lam, omega, rank, iters):
    N, K = w.shape
    p = omega.shape[1]
    l1t = torch.empty((rank, K), dtype=torch.bfloat16, device="cuda")
    l2t = torch.empty((N, rank), dtype=torch.bfloat16, device="cuda")
    res = torch.empty((N, K), dtype=torch.float32, device="cuda")
    st = sq.lib().svdq_lowrank_decompose_noalloc(
        N, K, rank, p - rank, iters, ctypes.c_void_p(w.data_ptr()), ctypes.c_void_p(lam.data_ptr()),
        ctypes.c_void_p(omega.data_ptr()), ctypes.c_void_p(l1t.data_ptr()), ctypes.c_void_p(l2t.data_ptr()),
        ctypes.c_void_p(res.data_ptr()), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, sq.lib().svdq_last_error()
    return l1t, l2t, res


def same(a, b):
    return torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32),
                       b.view(torch.int16) if b.dtype == torch.bfloat16 else b.view(torch.int32))


def test_noalloc_matches_the_allocating_entry_point():
    for N, K, rank, p, seed in ((1536, 768, 32, 48, 4101), (640, 384, 16, 32, 4102)):
        print(f"[noalloc] decompose {N}x{K} rank {rank} p {p}", flush=True)
        d = synth.dense_layer(seed, N, K, planted_rank=rank)
        lam = b16(oracle.calibrate_smooth(d["x_cal"], d["w"]))
        w, om = b16(d["w"]), dev(d["omega"][:, :p])
        a = noalloc(w, lam, om, rank, 4)
        b = sq.lowrank_decompose(w, lam, om, rank, iters=4)
        torch.cuda.synchronize()
        for x, y, name in zip(a, b, ("l1t", "l2t", "residual")):
            assert same(x, y), f"{name} differs from svdq_lowrank_decompose"
        assert torch.isfinite(a[2]).all()
