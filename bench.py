"""Benchmark of the SVDQuant W4A4 linear + AWQ W4A16 GEMV hot path on one MI355X.

One step = one pass of the whole hot path over one batch of synthetic input:
  1. svdq_quantize_act  on the DiT fused-QKV projection input X [4608, 3072]
     (smoothing, int4 group-64 codes and scales, fused X.L1 with rank 32),
  2. svdq_w4a4_gemm     against W [9216, 3072] (int4 group 64) with the fused
     low-rank up-projection and bias, Y bf16 [4608, 9216],
  3. awq_w4a16_gemv     on the modulation projection x [2, 3072] x W [18432, 3072].
Inputs are resident in HBM before timing starts; several copies of every input
are cycled so that the 256 MB Infinity Cache cannot serve a step from the
previous one.  `value` is whole-step throughput in tera-ops per second,
2*M*N*K of the W4A4 linear divided by the time of the full step.

Prints one JSON line.  --gpus above 1 exits: this build measures one GPU.
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "W4A4 SVDQ linear TOPS (M=4608,K=3072) + AWQ GEMV GB/s; % of roofline"
PEAK_INT8_TOPS = 5000.0   # MI355X dense int8 matrix peak, 5.0 POP/s
PEAK_HBM_GBS = 8000.0     # MI355X HBM3E, 8 TB/s


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--copies", type=int, default=4, help="input copies cycled for the linear")
    p.add_argument("--awq-copies", type=int, default=16, help="AWQ weight copies cycled (>= 512 MB)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-rows", type=int, default=768, help="rows of X in the oracle's timed sample")
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


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported by this build "
              "(each box has a single MI355X; see the sharding notes in DESIGN.md)", file=sys.stderr)
        sys.exit(2)

    import torch
    import bit_w4a4_quantized_smooth_amd as sq
    from bit_w4a4_quantized_smooth_amd import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    sq.lib()

    # ---- inputs ----------------------------------------------------------------
    M, N, K, R = 4608, 9216, 3072, 32
    lin = synth.svdq_layer(1002, M, N, K, R, synth.INT4, 0.005, 30.0)
    awq = synth.awq_layer(1005, 2, 18432, 3072)

    def t(a, dtype=None):
        x = torch.from_numpy(np.ascontiguousarray(a))
        return (x.view(dtype) if dtype is not None else x).to(dev)

    def bf(bits):
        return t(np.asarray(bits, np.uint16).view(np.int16), torch.bfloat16)

    def f16(bits):
        return t(np.asarray(bits, np.uint16).view(np.int16), torch.float16)

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

    A = max(1, args.awq_copies)
    AX = bf(awq["x"])
    AWC = [t(awq["w_codes"]) for _ in range(A)]
    AWS = [f16(awq["w_scales"]) for _ in range(A)]
    AWZ = [f16(awq["w_zeros"]) for _ in range(A)]
    ABIAS = bf(awq["bias"])
    AY = torch.empty((2, 18432), dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()

    def step(i, ev=None):
        c = i % C
        if ev is not None:
            ev[0].record(stream)
        sq.quantize_act(sq.SVDQ_INT4, X[c], LAM, L1T, out=(CODES[c], SCALES[c], XL1[c]), stream=stream)
        if ev is not None:
            ev[1].record(stream)
        sq.w4a4_gemm(sq.SVDQ_INT4, CODES[c], SCALES[c], WC[c], WS[c], XL1[c], L2T, BIAS, out=Y[i % 2],
                     stream=stream)
        if ev is not None:
            ev[2].record(stream)
        a = i % A
        sq.awq_gemv(AX, AWC[a], AWS[a], AWZ[a], ABIAS, out=AY, stream=stream)
        if ev is not None:
            ev[3].record(stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i, evs[i])
    torch.cuda.synchronize()
    wall_s = time.perf_counter() - t0

    t_quant = np.array([e[0].elapsed_time(e[1]) for e in evs])
    t_gemm = np.array([e[1].elapsed_time(e[2]) for e in evs])
    t_awq = np.array([e[2].elapsed_time(e[3]) for e in evs])
    t_step = np.array([e[0].elapsed_time(e[3]) for e in evs])
    ms_step = float(wall_s * 1e3 / args.steps)

    ops = 2.0 * M * N * K
    gemm_ms = float(t_gemm.mean())
    gemm_tops = ops / (gemm_ms * 1e-3) / 1e12
    quant_bytes = M * K * 2 + K * 2 + R * K * 2 + M * K // 2 + M * (K // 64) * 2 + M * R * 4
    awq_bytes = 18432 * 3072 // 2 + 2 * 18432 * 48 * 2 + 2 * 3072 * 2 + 18432 * 2 + 2 * 18432 * 2

    out = {
        "metric": METRIC,
        "value": round(ops / (ms_step * 1e-3) / 1e12, 2),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8",
        "data": "synthetic",
        "config": {"workload": "dit_qkv_int4_4608x9216x3072_r32 + awq_mod_2x18432x3072",
                   "M": M, "N": N, "K": K, "rank": R, "group": 64, "awq": [2, 18432, 3072]},
        "components": {
            "quantize_ms": round(float(t_quant.mean()), 5),
            "quantize_GBps": round(quant_bytes / (t_quant.mean() * 1e-3) / 1e9, 1),
            "gemm_ms": round(gemm_ms, 5),
            "gemm_TOPS": round(gemm_tops, 2),
            "linear_TOPS": round(ops / ((t_quant.mean() + gemm_ms) * 1e-3) / 1e12, 2),
            "awq_ms": round(float(t_awq.mean()), 5),
            "awq_GBps": round(awq_bytes / (t_awq.mean() * 1e-3) / 1e9, 1),
            "awq_frac_hbm": round(awq_bytes / (t_awq.mean() * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "event_step_ms": round(float(t_step.mean()), 5),
        },
        "roofline": {"bound": "mfma", "achieved": round(gemm_tops, 2), "peak": PEAK_INT8_TOPS,
                     "unit": "TFLOP/s", "frac": round(gemm_tops / PEAK_INT8_TOPS, 4), "traffic": None,
                     "kernel": "gemm_int4_kernel", "per_launch_ops": ops},
    }

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(lin, args.cpu_rows)
    print(json.dumps(out), flush=True)


def cpu_baseline(lin, rows):
    """The oracle, as it stands, on the first `rows` rows of the same workload:
    quantize + X.L1 + the full linear for those rows against all N columns."""
    import oracle
    nthreads = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    x = np.ascontiguousarray(lin["x"][:rows])
    t0 = time.perf_counter()
    codes, scales = oracle.quantize_act(oracle.INT4, x, lin["lam"], nthreads=nthreads)
    xl1 = oracle.lowrank_down(x, lin["l1t"], nthreads=nthreads)
    oracle.w4a4_linear(oracle.INT4, codes, scales, lin["w_codes"], lin["w_scales"], xl1, lin["l2t"],
                       lin["bias"], nthreads=nthreads)
    dt = time.perf_counter() - t0
    ops = 2.0 * rows * lin["N"] * lin["K"]
    return {"value": round(ops / dt / 1e12, 6), "unit": "TOPS", "cores": nthreads, "kind": "oracle",
            "sample": f"first {rows} of {lin['M']} rows of the linear (quantize + X.L1 + all "
                      f"{lin['N']} outputs), {dt:.2f} s"}


if __name__ == "__main__":
    main()
