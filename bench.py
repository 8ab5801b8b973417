"""Benchmark of the SVDQuant W4A4 linear + AWQ W4A16 GEMV hot path on one MI355X.

One step = one pass of the whole hot path over one batch of synthetic input:
  1. the quantizer on the DiT fused-QKV projection input X [4608, 3072]
     (smoothing, int4 group-64 codes and scales, fused X.L1 with rank 32),
  2. svdq_w4a4_gemm_ws  against W [9216, 3072] (int4 group 64) with the fused
     low-rank up-projection and bias, Y bf16 [4608, 9216] (with its workspace:
     the grid's last partial round of tiles runs as K slices),
  3. the AWQ GEMV on the modulation projection x [2, 3072] x W [18432, 3072].
Steps 1 and 3 do not depend on each other and go out as one launch,
svdq_quantize_act_awq_gemv (the GEMV's workgroups run on the CUs the
quantizer's 144 workgroups leave idle), then step 2; --no-fuse launches the
three separately (svdq_quantize_act_ws, svdq_w4a4_gemm_ws, awq_w4a16_gemv).
Inputs are resident in HBM before timing starts; several copies of every input
are cycled so that the 256 MB Infinity Cache cannot serve a step from the
previous one.  `value` is whole-step throughput in tera-ops per second,
2*M*N*K of the W4A4 linear divided by the time of the full step.

Besides the step, the same run times the other workloads of the hot path one
call at a time (median of timed calls, HIP events on the launch stream): the
DiT MLP up/down projections, the NVFP4 variant of the QKV projection, the
AWQ GEMV at M=64, and a plain device-to-device copy as the attainable-HBM
line.  `roofline` describes the dominant kernel (the int4 GEMM); its `traffic`
is the HBM bytes per launch from the committed FETCH_SIZE / WRITE_SIZE
counter summary, reported only while the kernel source still matches the
hash recorded there.

Prints one JSON line.  --gpus above 1 exits with a message: the benchmark runs on one GPU.
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "W4A4 SVDQ linear TOPS (M=4608,K=3072) + AWQ GEMV GB/s; % of roofline"
PEAK_INT8_TOPS = 5000.0   # MI355X dense int8 matrix peak, 5.0 POP/s
PEAK_FP8_TFLOPS = 5000.0  # dense fp8
PEAK_FP4_TFLOPS = 10100.0 # dense fp4 / fp6
PEAK_BF16_TFLOPS = 2500.0 # dense bf16
PEAK_HBM_GBS = 8000.0     # MI355X HBM3E, 8 TB/s
GEMM_SOURCES = ["gemm_int4.hip", "tail_split.h", "common.h", "launch.h"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_gemm_int4_dit_qkv_4608x9216x3072.txt")


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    # The GPU's clocks need tens of milliseconds of sustained load to settle
    # (a 4608x9216x3072 GEMM runs ~15% slower for the first ~40 ms after idle):
    # before the warm-up steps, untimed steps run until this much wall time has
    # passed with the GPU busy.  Reported in the JSON line as settle_ms and
    # settle_steps; 0 disables it.
    p.add_argument("--settle-ms", type=float, default=150.0)
    p.add_argument("--copies", type=int, default=4, help="input copies cycled for the linear")
    p.add_argument("--awq-copies", type=int, default=16, help="AWQ weight copies cycled (>= 512 MB)")
    p.add_argument("--calls", type=int, default=20, help="timed calls per extra workload")
    p.add_argument("--no-extras", action="store_true", help="time only the step")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-fuse", action="store_true",
                   help="launch the quantizer and the AWQ GEMV separately in the timed steps")
    p.add_argument("--cpu-rows", type=int, default=1152, help="rows of X in the oracle's timed sample")
    p.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                   help="instead of the benchmark, copy MIB MiB device-to-device a few times (the known-size "
                        "transfer that scales the FETCH_SIZE / WRITE_SIZE counters)")
    return p.parse_args()


def copy_calibration(mib):
    import torch
    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n, "launches": 3}), flush=True)


def gemm_source_hash():
    """SHA-256 of the GEMM's source code with // comments and blank lines
    removed, so that editing a comment does not invalidate the counters."""
    h = hashlib.sha256()
    for name in GEMM_SOURCES:
        with open(os.path.join(ROOT, "bit_w4a4_quantized_smooth_amd", "csrc", name)) as f:
            for line in f:
                code = line.split("//", 1)[0].rstrip()
                if code:
                    h.update(code.encode() + b"\n")
    return h.hexdigest()


def committed_traffic():
    """HBM bytes per launch of the int4 GEMM from the committed counter summary,
    or None when it is missing or was taken on a different kernel source."""
    try:
        fields = {}
        with open(TRAFFIC_FILE) as f:
            for line in f:
                if ":" in line and not line.startswith("#"):
                    k, v = line.split(":", 1)
                    fields[k.strip()] = v.strip()
        if fields.get("source_sha256") != gemm_source_hash():
            return None
        return int(fields["fetch_bytes_per_launch"]) + int(fields["write_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (the linear shards "
              "on tokens with no communication, so each GPU would repeat this one-GPU step)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import bit_w4a4_quantized_smooth_amd as sq
    from bit_w4a4_quantized_smooth_amd import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    sq.lib()

    def t(a, dtype=None):
        x = torch.from_numpy(np.ascontiguousarray(a))
        return (x.view(dtype) if dtype is not None else x).to(dev)

    def bf(bits):
        return t(np.asarray(bits, np.uint16).view(np.int16), torch.bfloat16)

    def f16(bits):
        return t(np.asarray(bits, np.uint16).view(np.int16), torch.float16)

    stream = torch.cuda.current_stream()

    # ---- the step: DiT QKV int4 linear + AWQ modulation GEMV --------------------
    M, N, K, R = 4608, 9216, 3072, 32
    lin = synth.svdq_layer(1002, M, N, K, R, synth.INT4, 0.005, 30.0)
    awq = synth.awq_layer(1005, 2, 18432, 3072)

    C = max(1, args.copies)
    X = [bf(lin["x"]) for _ in range(C)]
    LAM = bf(lin["lam"])
    L1T = bf(lin["l1t"])
    WC = [t(lin["w_codes"]) for _ in range(C)]
    WS = [f16(lin["w_scales"]) for _ in range(C)]
    L2T = bf(lin["l2t"])
    BIAS = bf(lin["bias"])
    CODES = [torch.empty((M, K // 2), dtype=torch.uint8, device=dev) for _ in range(C)]
    SCALES = [torch.empty((M, K // 64), dtype=torch.float16, device=dev) for _ in range(C)]
    XL1 = [torch.empty((M, R), dtype=torch.float32, device=dev) for _ in range(C)]
    Y = [torch.empty((M, N), dtype=torch.bfloat16, device=dev) for _ in range(2)]
    # one workspace for the stream: the quantizer's balanced split (svdq_quantize_act_ws)
    # and the GEMM's split last round of tiles (svdq_w4a4_gemm_ws)
    WORK = sq.gemm_workspace(dev)

    A = max(1, args.awq_copies)
    AX = bf(awq["x"])
    AWC = [t(awq["w_codes"]) for _ in range(A)]
    AWS = [f16(awq["w_scales"]) for _ in range(A)]
    AWZ = [f16(awq["w_zeros"]) for _ in range(A)]
    ABIAS = bf(awq["bias"])
    AY = torch.empty((2, 18432), dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()

    def step(i, ev=None, gemm_ev=None, fused=not args.no_fuse):
        # ev: events around every launch (component timing, untimed passes);
        # gemm_ev: events around the GEMM only (the timed steps: each event
        # record adds a small gap to the stream, so the timed steps carry two).
        # fused: the quantizer and the AWQ GEMV (independent of each other) go
        # out as one launch (svdq_quantize_act_awq_gemv), then the GEMM.
        c = i % C
        a = i % A
        if fused:
            if ev is not None:
                ev[0].record(stream)
            sq.quantize_act_awq_gemv(sq.SVDQ_INT4, X[c], LAM, L1T, 1.0, AX, AWC[a], AWS[a], AWZ[a], ABIAS,
                                     out=(CODES[c], SCALES[c], XL1[c]), awq_out=AY, stream=stream)
            if ev is not None:
                ev[1].record(stream)
            if gemm_ev is not None:
                gemm_ev[0].record(stream)
            sq.w4a4_gemm(sq.SVDQ_INT4, CODES[c], SCALES[c], WC[c], WS[c], XL1[c], L2T, BIAS, out=Y[i % 2],
                         stream=stream, workspace=WORK)
            if gemm_ev is not None:
                gemm_ev[1].record(stream)
            if ev is not None:
                ev[2].record(stream)
            return
        if ev is not None:
            ev[0].record(stream)
        sq.quantize_act(sq.SVDQ_INT4, X[c], LAM, L1T, out=(CODES[c], SCALES[c], XL1[c]), stream=stream,
                        workspace=WORK)
        if ev is not None:
            ev[1].record(stream)
        if gemm_ev is not None:
            gemm_ev[0].record(stream)
        sq.w4a4_gemm(sq.SVDQ_INT4, CODES[c], SCALES[c], WC[c], WS[c], XL1[c], L2T, BIAS, out=Y[i % 2],
                     stream=stream, workspace=WORK)
        if ev is not None:
            ev[2].record(stream)
        if gemm_ev is not None:
            gemm_ev[1].record(stream)
        sq.awq_gemv(AX, AWC[a], AWS[a], AWZ[a], ABIAS, out=AY, stream=stream)
        if ev is not None:
            ev[3].record(stream)

    settle_steps = 0
    if args.settle_ms > 0:
        t0 = time.perf_counter()
        while (time.perf_counter() - t0) * 1e3 < args.settle_ms:
            for _ in range(16):
                step(settle_steps)
                settle_steps += 1
            torch.cuda.synchronize()
    for i in range(args.warmup):
        step(settle_steps + i)
    torch.cuda.synchronize()

    gevs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(settle_steps + args.warmup + i, gemm_ev=gevs[i])
    torch.cuda.synchronize()
    wall_s = time.perf_counter() - t0
    t_gemm = np.array([e[0].elapsed_time(e[1]) for e in gevs])

    # component durations: further untimed passes with events around every
    # launch, one with the three kernels launched separately, one fused
    nc = min(args.steps, 50)
    base_i = settle_steps + args.warmup + args.steps
    for i in range(5):  # the kernels of the other mode load on their first launch: keep that out
        step(base_i + i, fused=args.no_fuse)
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(nc)]
    for i in range(nc):
        step(settle_steps + args.warmup + args.steps + i, evs[i], fused=False)
    torch.cuda.synchronize()
    t_quant = np.array([e[0].elapsed_time(e[1]) for e in evs])
    t_awq = np.array([e[2].elapsed_time(e[3]) for e in evs])
    t_step = np.array([e[0].elapsed_time(e[3]) for e in evs])
    fevs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(nc)]
    for i in range(nc):
        step(settle_steps + args.warmup + args.steps + nc + i, fevs[i], fused=True)
    torch.cuda.synchronize()
    t_fused = np.array([e[0].elapsed_time(e[1]) for e in fevs])
    t_fstep = np.array([e[0].elapsed_time(e[2]) for e in fevs])
    ms_step = float(wall_s * 1e3 / args.steps)

    ops = 2.0 * M * N * K
    gemm_ms = float(t_gemm.mean())  # mean, like the kernel-trace average it is checked against
    gemm_tops = ops / (gemm_ms * 1e-3) / 1e12
    quant_bytes = M * K * 2 + K * 2 + R * K * 2 + M * K // 2 + M * (K // 64) * 2 + M * R * 4
    awq_bytes = 18432 * 3072 // 2 + 2 * 18432 * 48 * 2 + 2 * 3072 * 2 + 18432 * 2 + 2 * 18432 * 2

    components = {
        "quantize_ms": round(float(t_quant.mean()), 5),
        "quantize_GBps": round(quant_bytes / (t_quant.mean() * 1e-3) / 1e9, 1),
        "gemm_ms": round(gemm_ms, 5),
        "gemm_TOPS": round(gemm_tops, 2),
        "linear_TOPS": round(ops / ((t_quant.mean() + gemm_ms) * 1e-3) / 1e12, 2),
        "awq_ms": round(float(t_awq.mean()), 5),
        "awq_GBps": round(awq_bytes / (t_awq.mean() * 1e-3) / 1e9, 1),
        "awq_frac_hbm": round(awq_bytes / (t_awq.mean() * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
        "event_step_ms": round(float(t_step.mean()), 5),
        "quantize_awq_fused_ms": round(float(t_fused.mean()), 5),
        "event_step_fused_ms": round(float(t_fstep.mean()), 5),
        "step_launches": ("quantize+awq fused (svdq_quantize_act_awq_gemv), gemm" if not args.no_fuse
                          else "quantize, gemm, awq"),
    }
    if not args.no_extras:
        components.update(extras(args, torch, sq, synth, t, bf, f16, stream))

    traffic = committed_traffic()
    out = {
        "metric": METRIC,
        "value": round(ops / (ms_step * 1e-3) / 1e12, 2),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_ms": args.settle_ms,
        "settle_steps": settle_steps,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8",
        "data": "synthetic",
        "config": {"workload": "dit_qkv_int4_4608x9216x3072_r32 + awq_mod_2x18432x3072",
                   "M": M, "N": N, "K": K, "rank": R, "group": 64, "awq": [2, 18432, 3072]},
        "components": components,
        "roofline": {"bound": "mfma", "achieved": round(gemm_tops, 2), "peak": PEAK_INT8_TOPS,
                     "unit": "TOPS", "frac": round(gemm_tops / PEAK_INT8_TOPS, 4), "traffic": traffic,
                     "kernel": "gemm_int4_kernel", "per_launch_ops": ops,
                     "algorithmic_bytes": int(M * K // 2 + M * K // 64 * 2 + N * K // 2 + N * K // 64 * 2
                                              + M * R * 4 + N * R * 2 + N * 2 + M * N * 2)},
    }

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(lin, args.cpu_rows, synth)
    print(json.dumps(out), flush=True)


def median_ms(fn, calls, stream, torch, settle_ms=150.0):
    """Median duration of `calls` back-to-back calls, each bracketed by HIP events
    on the launch stream, after untimed calls that keep the GPU busy for about
    settle_ms (its clocks settle under sustained load: the NVFP4 QKV GEMM, first
    timed after 50 ms of its own calls, read 294.5 us, and 270.2 us after 300 ms)."""
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    fn(0)
    b.record(stream)
    torch.cuda.synchronize()
    n_settle = int(min(2000, max(3, settle_ms / max(a.elapsed_time(b), 1e-3))))
    for _ in range(n_settle):
        fn(0)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(calls)]
    for i, (a, b) in enumerate(evs):
        a.record(stream)
        fn(i)
        b.record(stream)
    torch.cuda.synchronize()
    return float(np.median([a.elapsed_time(b) for a, b in evs]))


def extras(args, torch, sq, synth, t, bf, f16, stream):
    """The hot path's other workloads, one call at a time."""
    res = {}
    dev = torch.device("cuda:0")
    n = args.calls
    work = sq.gemm_workspace(dev)

    def linear(name, seed, M, N, K, prec, outlier_frac, outlier_scale, kind="normal"):
        d = synth.svdq_layer(seed, M, N, K, 32, prec, outlier_frac, outlier_scale, kind)
        G = 64 if prec == sq.SVDQ_INT4 else 16
        x, lam, l1t = bf(d["x"]), bf(d["lam"]), bf(d["l1t"])
        wc = t(d["w_codes"])
        ws = f16(d["w_scales"]) if prec == sq.SVDQ_INT4 else t(d["w_scales"])
        l2t, bias = bf(d["l2t"]), bf(d["bias"])
        codes = torch.empty((M, K // 2), dtype=torch.uint8, device=dev)
        scales = (torch.empty((M, K // G), dtype=torch.float16, device=dev) if prec == sq.SVDQ_INT4
                  else torch.empty((M, K // G), dtype=torch.uint8, device=dev))
        xl1 = torch.empty((M, 32), dtype=torch.float32, device=dev)
        y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        aa, aw = float(d["alpha_a"]), float(d["alpha_w"])
        q_ms = median_ms(lambda i: sq.quantize_act(prec, x, lam, l1t, aa, out=(codes, scales, xl1), stream=stream,
                                                   workspace=work), n, stream, torch)
        q0_ms = median_ms(lambda i: sq.quantize_act(prec, x, lam, l1t, aa, out=(codes, scales, xl1), stream=stream),
                          n, stream, torch)
        g_ms = median_ms(lambda i: sq.w4a4_gemm(prec, codes, scales, wc, ws, xl1, l2t, bias, aa, aw, out=y,
                                                stream=stream, workspace=work), n, stream, torch)
        ops = 2.0 * M * N * K
        tops = ops / (g_ms * 1e-3) / 1e12
        qb = M * K * 2 + K * 2 + 32 * K * 2 + M * K // 2 + M * (K // G) * (2 if prec == sq.SVDQ_INT4 else 1) + M * 32 * 4
        r = {"quantize_ms": round(q_ms, 5), "quantize_GBps": round(qb / (q_ms * 1e-3) / 1e9, 1),
             "quantize_no_workspace_ms": round(q0_ms, 5),
             "gemm_ms": round(g_ms, 5), "gemm_TOPS": round(tops, 2),
             "linear_TOPS": round(ops / ((q_ms + g_ms) * 1e-3) / 1e12, 2)}
        if prec == sq.SVDQ_INT4:
            r["gemm_frac_int8"] = round(tops / PEAK_INT8_TOPS, 4)
        else:
            r["gemm_frac_fp8"] = round(tops / PEAK_FP8_TFLOPS, 4)
            r["gemm_frac_fp4"] = round(tops / PEAK_FP4_TFLOPS, 4)
        res[name] = r
        del x, lam, l1t, wc, ws, l2t, bias, codes, scales, xl1, y

    linear("mlp_up_int4_4608x12288x3072", 1002, 4608, 12288, 3072, sq.SVDQ_INT4, 0.005, 30.0)
    linear("mlp_down_int4_4608x3072x12288", 1003, 4608, 3072, 12288, sq.SVDQ_INT4, 0.0, 1.0, "gelu")
    linear("qkv_nvfp4_4608x9216x3072", 1004, 4608, 9216, 3072, sq.SVDQ_NVFP4, 0.005, 30.0)

    # fused attention projection (QKV GEMM + per-head RMSNorm + rotary epilogue)
    # against the same GEMM followed by the norm and rotary steps as separate
    # torch kernels on the bf16 output (both GEMMs with the workspace)
    for name, seed, prec in (("qkv_fused_int4_4608x9216x3072_h24d128", 1002, sq.SVDQ_INT4),
                             ("qkv_fused_nvfp4_4608x9216x3072_h24d128", 1004, sq.SVDQ_NVFP4)):
        M, H, D, K = 4608, 24, 128, 3072
        HD, N = H * D, 3 * H * D
        d = synth.qkv_layer(seed, M, H, D, K, 32, prec, 0.005, 30.0)
        G = 64 if prec == sq.SVDQ_INT4 else 16
        x, lam, l1t = bf(d["x"]), bf(d["lam"]), bf(d["l1t"])
        wc = t(d["w_codes"])
        ws = f16(d["w_scales"]) if prec == sq.SVDQ_INT4 else t(d["w_scales"])
        l2t, bias = bf(d["l2t"]), bf(d["bias"])
        nq, nk, rope = bf(d["norm_q"]), bf(d["norm_k"]), t(d["rope"])
        aa, aw, eps = float(d["alpha_a"]), float(d["alpha_w"]), float(d["eps"])
        codes, scales, xl1 = sq.quantize_act(prec, x, lam, l1t, aa, stream=stream)
        y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        fused_ms = median_ms(lambda i: sq.w4a4_gemm_qkv_norm_rope(
            prec, codes, scales, wc, ws, xl1, l2t, bias, H, D, nq, nk, eps, rope, aa, aw, out=y, stream=stream,
            workspace=work), n, stream, torch)
        plain_ms = median_ms(lambda i: sq.w4a4_gemm(prec, codes, scales, wc, ws, xl1, l2t, bias, aa, aw, out=y,
                                                    stream=stream, workspace=work), n, stream, torch)
        cos, sin = rope[:, :, 0].unsqueeze(1), rope[:, :, 1].unsqueeze(1)

        def norm_rope(part, w):
            h = y[:, part * HD:(part + 1) * HD].view(M, H, D).float()
            h = h * torch.rsqrt(h.pow(2).mean(-1, keepdim=True) + eps) * w.float()
            a, b = h[..., 0::2], h[..., 1::2]
            y[:, part * HD:(part + 1) * HD] = torch.stack([a * cos - b * sin, a * sin + b * cos], -1).view(M, HD).to(
                torch.bfloat16)

        def unfused(i):
            sq.w4a4_gemm(prec, codes, scales, wc, ws, xl1, l2t, bias, aa, aw, out=y, stream=stream, workspace=work)
            norm_rope(0, nq)
            norm_rope(1, nk)

        unfused_ms = median_ms(unfused, n, stream, torch)
        res[name] = {"fused_ms": round(fused_ms, 5), "plain_gemm_ms": round(plain_ms, 5),
                     "unfused_torch_ms": round(unfused_ms, 5),
                     "epilogue_overhead": round(fused_ms / plain_ms, 4),
                     "speedup_vs_unfused": round(unfused_ms / fused_ms, 3)}
        del x, lam, l1t, wc, ws, l2t, bias, nq, nk, rope, codes, scales, xl1, y

    # fused MLP up-projection (GEMM + GELU + the down projection's quantization and
    # X.L1) against the same GEMM writing bf16, torch's GELU and the quantizer
    for name, prec in (("mlp_up_fused_int4_4608x12288x3072", sq.SVDQ_INT4),
                       ("mlp_up_fused_nvfp4_4608x12288x3072", sq.SVDQ_NVFP4)):
        d = synth.mlp_layer(1002, 4608, 12288, 3072, 32, prec)
        up, dn = d["up"], d["down"]
        M, N, K = 4608, 12288, 3072
        G = 64 if prec == sq.SVDQ_INT4 else 16
        sc = f16 if prec == sq.SVDQ_INT4 else t
        aa, aw, ao = float(up["alpha_a"]), float(up["alpha_w"]), float(dn["alpha_a"])
        codes, scales, xl1 = sq.quantize_act(prec, bf(up["x"]), bf(up["lam"]), bf(up["l1t"]), aa, stream=stream)
        wc, ws, l2t, bias = t(up["w_codes"]), sc(up["w_scales"]), bf(up["l2t"]), bf(up["bias"])
        lam_d, l1t_d = bf(dn["lam"]), bf(dn["l1t"])
        outs = (torch.empty((M, N // 2), dtype=torch.uint8, device=dev),
                torch.empty((M, N // G), dtype=torch.float16 if prec == sq.SVDQ_INT4 else torch.uint8, device=dev),
                torch.empty((M, 32), dtype=torch.float32, device=dev))
        y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        fused_ms = median_ms(lambda i: sq.w4a4_gemm_gelu_quant(
            codes, scales, wc, ws, xl1, l2t, bias, lam_d, l1t_d, out=outs, stream=stream, precision=prec,
            act_global_scale=aa, w_global_scale=aw, out_global_scale=ao), n, stream, torch)
        plain_ms = median_ms(lambda i: sq.w4a4_gemm(prec, codes, scales, wc, ws, xl1, l2t, bias, aa, aw, out=y,
                                                    stream=stream), n, stream, torch)

        def unfused(i):
            sq.w4a4_gemm(prec, codes, scales, wc, ws, xl1, l2t, bias, aa, aw, out=y, stream=stream)
            h = torch.nn.functional.gelu(y)
            sq.quantize_act(prec, h, lam_d, l1t_d, ao, out=outs, stream=stream)

        unfused_ms = median_ms(unfused, n, stream, torch)
        res[name] = {"fused_ms": round(fused_ms, 5), "plain_gemm_ms": round(plain_ms, 5),
                     "unfused_ms": round(unfused_ms, 5), "epilogue_overhead": round(fused_ms / plain_ms, 4),
                     "speedup_vs_unfused": round(unfused_ms / fused_ms, 3)}
        del codes, scales, xl1, wc, ws, l2t, bias, lam_d, l1t_d, outs, y

    # offline weight side at the QKV projection's size (9216 x 3072, rank 32) and the
    # AWQ modulation weight (18432 x 3072): one call each (they run once per checkpoint)
    d = synth.dense_layer(1006, 9216, 3072, Mc=4608)
    w, xc, om = bf(d["w"]), bf(d["x_cal"]), t(d["omega"])

    def once_ms(fn):
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b)

    lam = sq.calibrate_smooth(xc, w, stream=stream)
    cal_ms = once_ms(lambda: sq.calibrate_smooth(xc, w, out=lam, stream=stream))
    dec = {}
    dec_ms = once_ms(lambda: dec.update(r=sq.lowrank_decompose(w, lam, om, 32, iters=4, stream=stream)))
    resid = dec["r"][2]
    qw_ms = median_ms(lambda i: sq.quantize_weight(sq.SVDQ_INT4, resid, stream=stream), n, stream, torch)
    wa = bf(synth.dense_layer(1007, 18432, 3072, Mc=16, planted_rank=0)["w"])
    aq_ms = median_ms(lambda i: sq.awq_quantize_weight(wa, stream=stream), n, stream, torch)
    qw_bytes = 9216 * 3072 * 4 + 9216 * 3072 // 2 + 9216 * 48 * 2
    aq_bytes = 18432 * 3072 * 2 + 18432 * 3072 // 2 + 2 * 18432 * 48 * 2
    res["offline_weight_side"] = {
        "calibrate_ms_9216x3072_calib4608": round(cal_ms, 4),
        "lowrank_decompose_ms_9216x3072_r32_it4": round(dec_ms, 3),
        "quantize_weight_int4_ms": round(qw_ms, 5),
        "quantize_weight_int4_GBps": round(qw_bytes / (qw_ms * 1e-3) / 1e9, 1),
        "awq_quantize_18432x3072_ms": round(aq_ms, 5),
        "awq_quantize_GBps": round(aq_bytes / (aq_ms * 1e-3) / 1e9, 1)}
    del d, w, xc, om, lam, dec, resid, wa

    # AWQ at M=16 and M=64 (the streamed matrix-core kernel) over >= 512 MB of weight copies
    d = synth.awq_layer(1005, 64, 18432, 3072)
    A = max(1, args.awq_copies)
    wc = [t(d["w_codes"]) for _ in range(A)]
    ws = [f16(d["w_scales"]) for _ in range(A)]
    wz = [f16(d["w_zeros"]) for _ in range(A)]
    b = bf(d["bias"])
    for m in (16, 64):
        x = bf(d["x"][:m])
        y = torch.empty((m, 18432), dtype=torch.bfloat16, device=dev)
        ms = median_ms(lambda i: sq.awq_gemv(x, wc[i % A], ws[i % A], wz[i % A], b, out=y, stream=stream),
                       n, stream, torch)
        byts = 18432 * 3072 // 2 + 2 * 18432 * 48 * 2 + m * 3072 * 2 + 18432 * 2 + m * 18432 * 2
        res[f"awq_m{m}"] = {"ms": round(ms, 5), "GBps": round(byts / (ms * 1e-3) / 1e9, 1),
                            "frac_hbm": round(byts / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
    del wc, ws, wz

    # attainable HBM: a 1 GiB device-to-device copy (read + write)
    src = torch.ones(1 << 30, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    ms = median_ms(lambda i: dst.copy_(src), 5, stream, torch)
    res["copy_attainable_GBps"] = round(2 * (1 << 30) / (ms * 1e-3) / 1e9, 1)
    del src, dst

    # context, not this library: the vendor's dense GEMMs (hipBLASLt under torch) at the
    # QKV projection's shape, int8 x int8 -> int32 with the weight as [N, K] (no group
    # scales, no low-rank branch, no bias) and bf16 x bf16 -> bf16
    M, N, K = 4608, 9216, 3072
    a8 = torch.randint(-8, 8, (M, K), dtype=torch.int8, device=dev)
    w8 = torch.randint(-8, 8, (N, K), dtype=torch.int8, device=dev)
    ab = torch.randn(M, K, dtype=torch.bfloat16, device=dev)
    wb = torch.randn(N, K, dtype=torch.bfloat16, device=dev)
    ops = 2 * M * N * K
    ms8 = median_ms(lambda i: torch._int_mm(a8, w8.t()), n, stream, torch)
    msb = median_ms(lambda i: torch.mm(ab, wb.t()), n, stream, torch)
    res["library_gemm_4608x9216x3072"] = {
        "int8_int_mm_ms": round(ms8, 5), "int8_TOPS": round(ops / (ms8 * 1e-3) / 1e12, 1),
        "bf16_mm_ms": round(msb, 5), "bf16_TFLOPS": round(ops / (msb * 1e-3) / 1e12, 1)}
    return res


def cpu_baseline(lin, rows, synth):
    """The oracle, as it stands, on bounded samples of the workloads, on the host's
    cores: `value` is the QKV linear (quantize + X.L1 + the linear against all N
    columns) on its first `rows` rows; `per_workload` adds the small int4
    workload in full on one thread and on all, and the first rows of the MLP
    projections, the NVFP4 QKV projection and the AWQ modulation projections."""
    import oracle
    nthreads = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()

    def linear(d, r, nt):
        x = np.ascontiguousarray(d["x"][:r])
        t0 = time.perf_counter()
        codes, scales = oracle.quantize_act(d["prec"], x, d["lam"], alpha=d["alpha_a"], nthreads=nt)
        xl1 = oracle.lowrank_down(x, d["l1t"], nthreads=nt)
        oracle.w4a4_linear(d["prec"], codes, scales, d["w_codes"], d["w_scales"], xl1, d["l2t"], d["bias"],
                           alpha_a=d["alpha_a"], alpha_w=d["alpha_w"], nthreads=nt)
        dt = time.perf_counter() - t0
        ops = 2.0 * r * d["N"] * d["K"]
        return {"value": round(ops / dt / 1e12, 6), "unit": "TOPS", "threads": nt, "seconds": round(dt, 3),
                "sample": f"first {r} of {d['M']} rows"}

    res = linear(lin, rows, nthreads)
    per = {}
    small = synth.WORKLOADS["svdq_int4_256x512x512_r16"]()
    per["svdq_int4_256x512x512_r16_1thread"] = linear(small, small["M"], 1)
    per["svdq_int4_256x512x512_r16"] = linear(small, small["M"], nthreads)
    # row counts sized to a few seconds each (the NVFP4 oracle decodes E2M1 and
    # E4M3 per product, about four times the int4 cost per row)
    for name, r in (("dit_mlp_up_int4_4608x12288x3072_r32", 576), ("dit_mlp_down_int4_4608x3072x12288_r32", 576),
                    ("dit_qkv_nvfp4_4608x9216x3072_r32", 144)):
        per[name] = linear(synth.WORKLOADS[name](), r, nthreads)
    for name in ("awq_mod_2x18432x3072", "awq_mod_64x18432x3072"):
        d = synth.WORKLOADS[name]()
        t0 = time.perf_counter()
        oracle.awq_linear(d["x"], d["w_codes"], d["w_scales"], d["w_zeros"], d["bias"], nthreads=nthreads)
        dt = time.perf_counter() - t0
        byts = d["N"] * d["K"] // 2 + 2 * d["N"] * (d["K"] // 64) * 2 + d["M"] * d["K"] * 2 + d["N"] * 2 + d["M"] * d["N"] * 2
        per[name] = {"value": round(byts / dt / 1e9, 3), "unit": "GB/s", "threads": nthreads, "seconds": round(dt, 3),
                     "sample": "all rows"}
    return {"value": res["value"], "unit": "TOPS", "cores": nthreads, "kind": "oracle",
            "sample": f"first {rows} of {lin['M']} rows of the QKV linear (quantize + X.L1 + all {lin['N']} "
                      f"outputs), {res['seconds']:.2f} s", "per_workload": per}


if __name__ == "__main__":
    main()
