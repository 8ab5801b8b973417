"""svdq_quantize_act_awq_gemv: the activation quantizer (blog "Nunchaku 4-bit
inference in Diffusers", "Background: SVDQuant and Nunchaku") and an
independent AWQ W4A16 projection ("Nunchaku Lite", "Supported quantization
types": awq_w4a16; blog, "Introducing Nunchaku Lite") in one launch, through
the C ABI.

Every output must be bit-identical to the two separate calls (svdq_quantize_act,
then awq_w4a16_gemv), and against the oracle: codes and scales bit-exact, XL1
within 1e-4 (normalized by its largest magnitude), the AWQ y within 1e-2
max-abs-rel.  Shapes: the DiT QKV input beside the modulation projection (one
launch), nvfp4 and rank 16 with one and four AWQ rows, a ragged quantizer, and
the shapes that fall back to two launches (rank 0, the chunked reciprocal
table, a GEMV with more rows), empty jobs, and poisoned guard bytes around
every output of a fused call.
"""
import numpy as np
import pytest
import torch

import oracle
import bit_w4a4_quantized_smooth_amd as sq
from bit_w4a4_quantized_smooth_amd import synth

pytestmark = pytest.mark.gpu

# (quantizer: precision, M, K, rank; AWQ: M, N, K)
CASES = [((sq.SVDQ_INT4, 4608, 3072, 32), (2, 18432, 3072)),   # the bench step's pair: one launch
         ((sq.SVDQ_NVFP4, 4608, 3072, 32), (1, 9216, 3072)),
         ((sq.SVDQ_INT4, 4100, 2048, 16), (4, 4096, 4096)),
         ((sq.SVDQ_NVFP4, 4200, 1024, 16), (3, 2048, 512)),
         ((sq.SVDQ_INT4, 4608, 3072, 0), (2, 4096, 3072)),      # rank 0: two launches
         ((sq.SVDQ_INT4, 4160, 12288, 32), (2, 4096, 3072)),    # chunked table: two launches
         ((sq.SVDQ_INT4, 4608, 3072, 32), (16, 4096, 3072)),    # GEMV of 16 rows: two launches
         ((sq.SVDQ_INT4, 300, 1024, 32), (2, 4096, 1024))]      # few quantizer rows: two launches


def b16(bits, dtype=torch.bfloat16):
    if bits is None:
        return None
    return torch.from_numpy(np.ascontiguousarray(np.asarray(bits, np.uint16).view(np.int16))).view(dtype).cuda()


def host(t):
    t = t.cpu()
    return t.view(torch.int16).numpy().view(np.uint16) if t.dtype in (torch.bfloat16, torch.float16) else t.numpy()


def inputs(q, a, seed):
    prec, M, K, r = q
    aM, aN, aK = a
    d = synth.svdq_layer(seed, M, 128, K, r, prec, 0.01, 25.0)
    w = synth.awq_layer(seed + 1, aM, aN, aK)
    qi = (prec, b16(d["x"]), b16(d["lam"]), b16(d["l1t"]) if r else None, d["alpha_a"])
    ai = (b16(w["x"]), torch.from_numpy(w["w_codes"]).cuda(), b16(w["w_scales"], torch.float16),
          b16(w["w_zeros"], torch.float16), b16(w["bias"]))
    return d, w, qi, ai


@pytest.mark.parametrize("q,a", CASES)
def test_fused_equals_separate_and_oracle(q, a):
    print(f"[quant_awq] quantizer {q} AWQ {a}", flush=True)
    d, w, qi, ai = inputs(q, a, 900 + q[1] % 89)
    (c, s, xl1), y = sq.quantize_act_awq_gemv(*qi, *ai)
    c0, s0, x0 = sq.quantize_act(*qi)
    y0 = sq.awq_gemv(*ai)
    torch.cuda.synchronize()
    assert np.array_equal(host(c), host(c0)) and np.array_equal(host(s), host(s0))
    assert (xl1 is None) == (x0 is None)
    if xl1 is not None:
        assert np.array_equal(host(xl1).view(np.uint32), host(x0).view(np.uint32)), "XL1 differs from the plain call"
    assert np.array_equal(host(y), host(y0)), "AWQ y differs from its own call"
    oc, os_ = oracle.quantize_act(q[0], d["x"], d["lam"], alpha=d["alpha_a"])
    assert np.array_equal(host(c), oc) and np.array_equal(host(s), os_)
    if q[3]:
        ox = oracle.lowrank_down(d["x"], d["l1t"])
        assert np.max(np.abs(host(xl1) - ox)) <= 1e-4 * np.max(np.abs(ox))
    ref, _ = oracle.awq_linear(w["x"], w["w_codes"], w["w_scales"], w["w_zeros"], w["bias"])
    err = float(np.max(np.abs(synth.bf16_bits_to_f64(host(y)) - ref)) / np.max(np.abs(ref)))
    print(f"[quant_awq] AWQ y max-abs-rel {err:.2e}", flush=True)
    assert err <= 1e-2


def test_empty_jobs():
    d, w, qi, ai = inputs((sq.SVDQ_INT4, 4608, 3072, 32), (2, 4096, 3072), 950)
    e = torch.empty((0, 3072), dtype=torch.bfloat16, device="cuda")
    (c, s, xl1), y = sq.quantize_act_awq_gemv(qi[0], e, qi[2], qi[3], qi[4], *ai)
    y0 = sq.awq_gemv(*ai)
    (c2, s2, x2), y2 = sq.quantize_act_awq_gemv(*qi, e[:, :3072], *ai[1:])
    c0, s0, x0 = sq.quantize_act(*qi)
    torch.cuda.synchronize()
    assert c.shape == (0, 1536) and np.array_equal(host(y), host(y0))
    assert y2.shape == (0, 4096) and np.array_equal(host(c2), host(c0)) and np.array_equal(host(x2), host(x0))


GUARD, POISON = 4096, 0xA5


def guarded(shape, dtype):
    n = int(np.prod(shape)) * torch.empty((), dtype=dtype).element_size()
    buf = torch.full((GUARD + n + GUARD,), POISON, dtype=torch.uint8, device="cuda")
    return buf, buf[GUARD:GUARD + n].view(dtype).view(shape), n


def test_fused_guards():
    # a ragged quantizer (4130 rows) and a GEMV of three rows, outputs inside poison
    q, a = (sq.SVDQ_INT4, 4130, 2048, 32), (3, 4096, 2048)
    d, w, qi, ai = inputs(q, a, 960)
    outs = [guarded((4130, 1024), torch.uint8), guarded((4130, 32), torch.float16), guarded((4130, 32), torch.float32),
            guarded((3, 4096), torch.bfloat16)]
    sq.quantize_act_awq_gemv(*qi, *ai, out=(outs[0][1], outs[1][1], outs[2][1]), awq_out=outs[3][1])
    torch.cuda.synchronize()
    for buf, _, n in outs:
        b = buf.cpu().numpy()
        assert (b[:GUARD] == POISON).all() and (b[GUARD + n:] == POISON).all(), "guard bytes overwritten"
    oc, os_ = oracle.quantize_act(q[0], d["x"], d["lam"], alpha=d["alpha_a"])
    assert np.array_equal(host(outs[0][1]), oc) and np.array_equal(host(outs[1][1]), os_)
    ref, _ = oracle.awq_linear(w["x"], w["w_codes"], w["w_scales"], w["w_zeros"], w["bias"])
    assert np.max(np.abs(synth.bf16_bits_to_f64(host(outs[3][1])) - ref)) <= 1e-2 * np.max(np.abs(ref))
