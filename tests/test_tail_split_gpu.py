"""svdq_w4a4_gemm_ws: the 4-bit GEMM with its grid's last partial round of
tiles run as K slices that meet in a caller-owned workspace.

On the QKV projection in int4 and in nvfp4 (4608 x 9216 x 3072, rank 32;
2592 tiles, so 32 tiles are left for the last round on a 256-CU device),
through the C ABI:
  * every output outside the split tiles is bit-identical to svdq_w4a4_gemm's;
  * the split ran: the partial tiles were written into the (zero-filled)
    workspace;
  * the split tiles match the oracle's double y (max-abs-rel <= 1e-2): two of
    them in full, 256 seeded outputs of each of the others (in nvfp4 the
    fp32 sums of these inputs are exact, multiples of 1/4 far below 2^24
    quanta, so there they equal svdq_w4a4_gemm's bit for bit; in int4 the
    constant offset of the integer-to-float step rounds, and some differ);
  * a second call gives the same bits, and every call leaves the counter
    words of the workspace zero;
  * a different activation through the same workspace is again right (no
    partial of the previous call is read);
  * where no split applies (a grid without a small last round), the result
    is svdq_w4a4_gemm's, bit for bit, and the workspace is not written.
The product is the blog's "Background: SVDQuant and Nunchaku" per-group
scaled 4-bit GEMM with the low-rank branch and bias in the epilogue.
"""
import numpy as np
import pytest
import torch

import oracle
import bit_w4a4_quantized_smooth_amd as sq
from bit_w4a4_quantized_smooth_amd import synth

pytestmark = pytest.mark.gpu

Y_TOL = 1e-2
TILE = 128
PART_BYTES = 16 * 1024 * 1024  # the counters follow the partial tiles


def dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    return (t.view(dtype) if dtype is not None else t).cuda()


def b16(bits, dtype=torch.bfloat16):
    return None if bits is None else dev(np.asarray(bits, np.uint16).view(np.int16), dtype)


def host(t):
    t = t.cpu()
    return t.view(torch.int16).numpy().view(np.uint16) if t.dtype in (torch.bfloat16, torch.float16) else t.numpy()


def split_tiles(prec, M, N, K, cus):
    """(row0, col0) of the tiles the launcher runs as K slices: the grid's tiles
    left after whole rounds of two per CU, when they are at most an eighth of a
    round, taken as the last tail/8 of each XCD's eighth of the banded tile order
    (int4: K of at least eight 128-channel stages; nvfp4: K a multiple of 1024
    channels, at least two such blocks)."""
    mt, nt = (M + TILE - 1) // TILE, N // TILE
    tiles, slots = mt * nt, 2 * cus
    k_ok = (K // 64 + 1) // 2 >= 8 if prec == sq.SVDQ_INT4 else (K // 64) % 16 == 0 and K // 1024 >= 2
    if tiles % 8 or slots % 8 or tiles <= slots or not k_ok:
        return []
    tail = tiles % slots
    if tail == 0 or tail > slots // 8 or tail > 64:
        return []
    tpx, tail_px, band_rows = tiles // 8, tail // 8, 12
    out = []
    for x in range(8):
        for tt in range(tail_px):
            t = x * tpx + tpx - tail_px + tt
            band = t // (band_rows * nt)
            in_band = t - band * band_rows * nt
            band_h = min(band_rows, mt - band * band_rows)
            out.append(((band * band_rows + in_band % band_h) * TILE, (in_band // band_h) * TILE))
    return out


def max_abs_rel(y_bits, ref):
    y = synth.bf16_bits_to_f64(y_bits)
    return float(np.max(np.abs(y - ref)) / max(np.max(np.abs(ref)), 1e-30))


def gemm(d, g, codes, scales, ws=None):
    return sq.w4a4_gemm(d["prec"], codes, scales, g["wc"], g["ws"], g["xl1"], g["l2t"], g["bias"], d["alpha_a"],
                        d["alpha_w"], workspace=ws)


def check_tiles(d, oc, os_, ox, y, tiles, full, seed):
    rng = np.random.default_rng(seed)
    for i, (m0, n0) in enumerate(tiles):
        rr, cc = np.meshgrid(np.arange(m0, m0 + TILE), np.arange(n0, n0 + TILE), indexing="ij")
        rr, cc = rr.ravel(), cc.ravel()
        if i >= full:
            pick = rng.choice(rr.size, 256, replace=False)
            rr, cc = rr[pick], cc[pick]
        ref, _ = oracle.w4a4_linear(d["prec"], oc, os_, d["w_codes"], d["w_scales"], ox, d["l2t"], d["bias"],
                                    alpha_a=d["alpha_a"], alpha_w=d["alpha_w"], rows=rr, cols=cc)
        e = max_abs_rel(y[rr, cc], ref)
        assert e <= Y_TOL, f"tile ({m0}, {n0}): max-abs-rel {e:.2e}"


@pytest.fixture(scope="module", params=["dit_qkv_int4_4608x9216x3072_r32", "dit_qkv_nvfp4_4608x9216x3072_r32"])
def qkv(request):
    name = request.param
    print(f"[tail split] {name}: inputs", flush=True)
    d = synth.WORKLOADS[name]()
    ws = b16(d["w_scales"], torch.float16) if d["prec"] == sq.SVDQ_INT4 else dev(d["w_scales"])
    g = dict(x=b16(d["x"]), lam=b16(d["lam"]), l1t=b16(d["l1t"]), wc=dev(d["w_codes"]), ws=ws,
             l2t=b16(d["l2t"]), bias=b16(d["bias"]))
    yield d, g
    del g
    torch.cuda.empty_cache()


def test_split_tail_on_the_qkv_projection(qkv):
    d, g = qkv
    M, N, K = d["M"], d["N"], d["K"]
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    tiles = split_tiles(d["prec"], M, N, K, cus)
    print(f"[tail split] {cus} CUs: {len(tiles)} tiles split", flush=True)
    if not tiles:
        pytest.skip(f"no split on a {cus}-CU device for this grid")
    codes, scales, xl1 = sq.quantize_act(d["prec"], g["x"], g["lam"], g["l1t"], d["alpha_a"])
    g["xl1"] = xl1
    work = sq.gemm_workspace()
    print("[tail split] plain GEMM, then twice with the workspace", flush=True)
    y_plain = gemm(d, g, codes, scales)
    y_ws = gemm(d, g, codes, scales, work)
    torch.cuda.synchronize()
    assert int(work[:PART_BYTES].count_nonzero()) > 0, "no partial tile written: no split ran"
    y_ws2 = gemm(d, g, codes, scales, work)
    torch.cuda.synchronize()
    assert torch.equal(y_ws.view(torch.int16), y_ws2.view(torch.int16)), "second call differs"
    assert int(work[PART_BYTES:].count_nonzero()) == 0, "counter words not left zero"

    in_split = torch.zeros((M, N), dtype=torch.bool, device="cuda")
    for m0, n0 in tiles:
        in_split[m0:m0 + TILE, n0:n0 + TILE] = True
    differ = y_ws.view(torch.int16) != y_plain.view(torch.int16)
    assert not bool((differ & ~in_split).any()), "outputs outside the split tiles differ"
    print(f"[tail split] {int(differ.sum())} outputs of the split tiles differ from the plain GEMM's", flush=True)

    oc, os_ = host(codes), host(scales)
    ox = oracle.lowrank_down(d["x"], d["l1t"])
    check_tiles(d, oc, os_, ox, host(y_ws), tiles, 2, 3)
    print("[tail split] split tiles match the oracle", flush=True)

    # a different activation (rows rotated) through the same workspace
    x2 = np.ascontiguousarray(np.roll(d["x"], 37, axis=0))
    codes2, scales2, xl12 = sq.quantize_act(d["prec"], b16(x2), g["lam"], g["l1t"], d["alpha_a"])
    g["xl1"] = xl12
    y2 = gemm(d, g, codes2, scales2, work)
    torch.cuda.synchronize()
    assert int(work[PART_BYTES:].count_nonzero()) == 0
    ox2 = oracle.lowrank_down(x2, d["l1t"])
    check_tiles(d, host(codes2), host(scales2), ox2, host(y2), tiles, 2, 5)
    print("[tail split] second activation through the same workspace matches the oracle", flush=True)


@pytest.mark.parametrize("name", ["svdq_int4_256x512x512_r16", "dit_mlp_up_int4_4608x12288x3072_r32"])
def test_no_split_is_the_plain_gemm(name):
    d = synth.WORKLOADS[name]()
    print(f"[tail split] {name}: with and without the workspace", flush=True)
    prec = d["prec"]
    sc = (lambda s: b16(s, torch.float16)) if prec == sq.SVDQ_INT4 else dev
    g = dict(wc=dev(d["w_codes"]), ws=sc(d["w_scales"]), l2t=b16(d["l2t"]), bias=b16(d["bias"]))
    codes, scales, g["xl1"] = sq.quantize_act(prec, b16(d["x"]), b16(d["lam"]), b16(d["l1t"]), d["alpha_a"])
    y0 = sq.w4a4_gemm(prec, codes, scales, g["wc"], g["ws"], g["xl1"], g["l2t"], g["bias"], d["alpha_a"], d["alpha_w"])
    work = sq.gemm_workspace()
    y1 = sq.w4a4_gemm(prec, codes, scales, g["wc"], g["ws"], g["xl1"], g["l2t"], g["bias"], d["alpha_a"], d["alpha_w"],
                      workspace=work)
    torch.cuda.synchronize()
    assert torch.equal(y0.view(torch.int16), y1.view(torch.int16))
    assert int(work.count_nonzero()) == 0


# Grids at the edges of the split: the smallest last round (8 tiles: 65 x 8
# tiles of 128 x 128) and the largest (64 tiles: 72 x 8), and the shortest K
# that is split (int4: eight 128-channel stages; nvfp4: two 1024-channel
# blocks).  Seeded synthetic layers of the same recipe as the workloads.
EDGES = [(sq.SVDQ_INT4, 8320, 1024, 1024), (sq.SVDQ_INT4, 9216, 1024, 2048),
         (sq.SVDQ_NVFP4, 8320, 1024, 2048), (sq.SVDQ_NVFP4, 9216, 1024, 2048)]


@pytest.mark.parametrize("prec,M,N,K", EDGES)
def test_split_tail_edges(prec, M, N, K):
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    tiles = split_tiles(prec, M, N, K, cus)
    print(f"[tail split] edge prec {prec} {M}x{N}x{K}: {len(tiles)} tiles split", flush=True)
    if not tiles:
        pytest.skip(f"no split on a {cus}-CU device for this grid")
    d = synth.svdq_layer(81 + M % 7 + K % 5, M, N, K, 16, prec, 0.005, 30.0)
    sc = (lambda s: b16(s, torch.float16)) if prec == sq.SVDQ_INT4 else dev
    g = dict(wc=dev(d["w_codes"]), ws=sc(d["w_scales"]), l2t=b16(d["l2t"]), bias=b16(d["bias"]))
    codes, scales, g["xl1"] = sq.quantize_act(prec, b16(d["x"]), b16(d["lam"]), b16(d["l1t"]), d["alpha_a"])
    work = sq.gemm_workspace()
    y_plain = gemm(d, g, codes, scales)
    y_ws = gemm(d, g, codes, scales, work)
    torch.cuda.synchronize()
    assert int(work[:PART_BYTES].count_nonzero()) > 0, "no partial tile written: no split ran"
    assert int(work[PART_BYTES:].count_nonzero()) == 0
    y_ws2 = gemm(d, g, codes, scales, work)
    torch.cuda.synchronize()
    assert torch.equal(y_ws.view(torch.int16), y_ws2.view(torch.int16))
    in_split = torch.zeros((M, N), dtype=torch.bool, device="cuda")
    for m0, n0 in tiles:
        in_split[m0:m0 + TILE, n0:n0 + TILE] = True
    differ = y_ws.view(torch.int16) != y_plain.view(torch.int16)
    assert not bool((differ & ~in_split).any()), "outputs outside the split tiles differ"
    xl1 = oracle.lowrank_down(d["x"], d["l1t"])
    check_tiles(d, host(codes), host(scales), xl1, host(y_ws), tiles, 1, 9)


@pytest.mark.parametrize("prec", [sq.SVDQ_INT4, sq.SVDQ_NVFP4])
def test_split_tail_fused_attention_projection(prec):
    # svdq_w4a4_gemm_qkv_norm_rope_ws on the 24-head x 128 QKV projection of the
    # same size: the last slice of a split tile runs the per-head RMSNorm and
    # rotary epilogue on the summed tile.  Outside the split tiles the output
    # equals svdq_w4a4_gemm_qkv_norm_rope's bit for bit; whole token rows through
    # the split tiles (the first row of each, every column, so every head whole)
    # match the oracle's projection per Q, K and V block within 1e-2.
    print(f"[tail split] fused attention projection prec {prec}", flush=True)
    d = synth.qkv_layer(1002 if prec == sq.SVDQ_INT4 else 1004, 4608, 24, 128, 3072, 32, prec, 0.005, 30.0)
    M, N, K, HD = 4608, 9216, 3072, 24 * 128
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    tiles = split_tiles(prec, M, N, K, cus)
    if not tiles:
        pytest.skip(f"no split on a {cus}-CU device for this grid")
    sc = (lambda s: b16(s, torch.float16)) if prec == sq.SVDQ_INT4 else dev
    codes, scales, xl1 = sq.quantize_act(prec, b16(d["x"]), b16(d["lam"]), b16(d["l1t"]), d["alpha_a"])
    args = (prec, codes, scales, dev(d["w_codes"]), sc(d["w_scales"]), xl1, b16(d["l2t"]), b16(d["bias"]), 24, 128,
            b16(d["norm_q"]), b16(d["norm_k"]), d["eps"], dev(d["rope"]), d["alpha_a"], d["alpha_w"])
    work = sq.gemm_workspace()
    y_plain = sq.w4a4_gemm_qkv_norm_rope(*args)
    y_ws = sq.w4a4_gemm_qkv_norm_rope(*args, workspace=work)
    torch.cuda.synchronize()
    assert int(work[:PART_BYTES].count_nonzero()) > 0, "no partial tile written: no split ran"
    assert int(work[PART_BYTES:].count_nonzero()) == 0
    in_split = torch.zeros((M, N), dtype=torch.bool, device="cuda")
    for m0, n0 in tiles:
        in_split[m0:m0 + TILE, n0:n0 + TILE] = True
    differ = y_ws.view(torch.int16) != y_plain.view(torch.int16)
    assert not bool((differ & ~in_split).any()), "outputs outside the split tiles differ"
    rows = np.unique([m0 for m0, _ in tiles])
    oc, os_ = host(codes), host(scales)
    ox = oracle.lowrank_down(d["x"], d["l1t"])
    ref, _ = oracle.w4a4_linear_qkv(prec, oc, os_, d["w_codes"], d["w_scales"], ox, d["l2t"], d["bias"], 24, 128,
                                    d["norm_q"], d["norm_k"], d["eps"], d["rope"], d["alpha_a"], d["alpha_w"],
                                    rows=rows)
    got = synth.bf16_bits_to_f64(host(y_ws)[rows])
    for b, name in enumerate("QKV"):
        g, r = got[:, b * HD:(b + 1) * HD], ref[:, b * HD:(b + 1) * HD]
        err = np.max(np.abs(g - r)) / max(np.max(np.abs(r)), 1e-30)
        print(f"[tail split] fused {name} block on {rows.size} rows through the split tiles: {err:.2e}", flush=True)
        assert err <= Y_TOL, f"{name} block: max-abs-rel {err:.3g}"
