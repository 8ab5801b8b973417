"""Mutation check of the oracle's pins (test infrastructure, CPU only).

Each mutant is the oracle's C++ source with one plausible slip planted in it:
a dropped factor, a wrong sign, a transposed operand or index, a wrong
rounding mode, a wrong format constant.  Every mutant is built with the
oracle's own compiler flags and the oracle's pin tests are run against it
(through SVDQ_ORACLE_LIB, in a subprocess of its own); each mutant must fail
at least one pin.  A mutant that passes them all names a slip the pins
cannot see.  The unmutated source, built and run the same way, must pass:
that is the control that the harness itself works.

Only slips that change some exported result are listed.  A slip that cannot
change any result (for instance the clamp of an int4 code at -8, which the
scale a/7 never reaches) is not a gap in the pins and is not listed.
"""
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
from oracle import build as oracle_build  # noqa: E402

PIN_TESTS = ("test_oracle_converters.py", "test_oracle_method.py", "test_oracle_mlp.py", "test_oracle_qkv.py",
             "test_oracle_offline.py")

# (name, text in the oracle source, replacement); the text must occur exactly once.
MUTANTS = [
    # number formats ("Supported quantization types": fp16/bf16 scales and
    # data, E4M3 scales and E2M1 values of NVFP4)
    ("round_half_away_from_zero", "std::nearbyint(a / quantum)", "std::round(a / quantum)"),
    ("round_toward_zero", "std::nearbyint(a / quantum)", "std::trunc(a / quantum)"),
    ("bf16_saturates", "return (uint16_t)encode(round_to_format(x, kBF16, false), kBF16, 8);\n}\ninline uint16_t f64",
     "return (uint16_t)encode(round_to_format(x, kBF16, true), kBF16, 8);\n}\ninline uint16_t f64"),
    ("f16_emin", "{10, -14, 65504.0", "{10, -15, 65504.0"),
    ("e4m3_max_of_ieee_variant", "{3, -6, 448.0, kFnNan}", "{3, -6, 240.0, kFnNan}"),
    ("e4m3_emin", "{3, -6, 448.0", "{3, -7, 448.0"),
    ("e2m1_emin", "{1, 0, 6.0, kNone}", "{1, 1, 6.0, kNone}"),
    # packing
    ("nibble_unsigned", "(n & 8) ? (int)(n & 0xF) - 16", "(n & 8) ? (int)(n & 0xF)"),
    ("nibble_order_on_read", "return (k & 1) ? (uint8_t)(b >> 4) : (uint8_t)(b & 0xF);",
     "return (k & 1) ? (uint8_t)(b & 0xF) : (uint8_t)(b >> 4);"),
    # smoothing ("Smoothing": the activation is divided by lambda)
    ("smoothing_multiplies", "r[k] = 1.0f / bf16_to_f32(lam[k]);", "r[k] = bf16_to_f32(lam[k]);"),
    # activation quantizers
    ("int4_act_scale_over_8", "      uint16_t sbits = f32_to_f16_sat(a / 7.0f);\n      scales[m * ng + g] = sbits;",
     "      uint16_t sbits = f32_to_f16_sat(a / 8.0f);\n      scales[m * ng + g] = sbits;"),
    ("int4_act_truncates", "          float r = std::nearbyint(v);", "          float r = std::trunc(v);"),
    ("nvfp4_act_scale_over_4", "const float d = 6.0f * alpha;", "const float d = 4.0f * alpha;"),
    ("nvfp4_act_drops_global_scale", "float sa = s * alpha; t = 1.0f / sa;", "float sa = s; t = 1.0f / sa;"),
    # low-rank down-projection ("Low-rank branch": XL1 = X L1)
    ("lowrank_down_transposed", "acc += xd[k] * lr[k];", "acc += xd[k] * l1d[(size_t)k * r + j];"),
    # the quantized linear
    ("linear_drops_weight_scale", "main += sa * sw * P;", "main += sa * P;"),
    ("linear_drops_weight_global_scale", "main *= (double)alpha_a * (double)alpha_w;", "main *= (double)alpha_a;"),
    ("linear_lowrank_sign", "return main + lr + b;", "return main - lr + b;"),
    ("linear_lowrank_up_transposed", "(double)bf16_to_f32(l2t[n * r + j])", "(double)bf16_to_f32(l2t[j * N + n])"),
    ("linear_drops_bias", "double b = bias ? (double)bf16_to_f32(bias[n]) : 0.0;", "double b = 0.0;"),
    # weight quantizers (offline)
    ("int4_weight_scale_over_8", "const uint16_t sbits = f32_to_f16_sat(a / 7.0f);",
     "const uint16_t sbits = f32_to_f16_sat(a / 8.0f);"),
    ("nvfp4_weight_drops_global_scale", "1.0f / (s * alpha);", "1.0f / s;"),
    # AWQ W4A16
    ("awq_zero_point_sign", "* (q - z) * s;", "* (q + z) * s;"),
    ("awq_drops_bias", "if (bias) acc += (double)bf16_to_f32(bias[n]);", ""),
    ("awq_scale_over_16", "(hi - lo) / 15.0f", "(hi - lo) / 16.0f"),
    ("awq_zero_point_sign_in_quantizer", "std::nearbyint(-lo * t)", "std::nearbyint(lo * t)"),
    # epilogues: GELU of the MLP, RMSNorm and RoPE of the attention heads
    ("gelu_without_sqrt2", "std::erfc(-y[i] / std::sqrt(2.0))", "std::erfc(-y[i] / 2.0)"),
    ("gelu_sign", "std::erfc(-y[i] / std::sqrt(2.0))", "std::erfc(y[i] / std::sqrt(2.0))"),
    ("rmsnorm_sum_not_mean", "std::sqrt(ss / D + eps)", "std::sqrt(ss + eps)"),
    ("rope_rotation_sign", "head[2 * p] = a * c - b * sn;", "head[2 * p] = a * c + b * sn;"),
]


def _build_and_pin(tmp, name, source):
    src = os.path.join(tmp, f"{name}.cpp")
    lib = os.path.join(tmp, f"lib{name}.so")
    with open(src, "w") as f:
        f.write(source)
    subprocess.run(["g++", "-O2", "-std=c++17", "-ffp-contract=off", "-fno-fast-math", "-shared", "-fPIC",
                    "-pthread", src, "-o", lib], check=True, timeout=300, capture_output=True)
    env = dict(os.environ, SVDQ_ORACLE_LIB=lib, OMP_NUM_THREADS="1")
    tests = [os.path.join(ROOT, "tests", t) for t in PIN_TESTS]
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu"]
                       + tests, cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    return name, r.returncode, r.stdout[-1500:]


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not found")
def test_every_mutant_fails_a_pin(tmp_path):
    with open(oracle_build.SRC) as f:
        base = f.read()
    jobs = [("control", base)]
    for name, old, new in MUTANTS:
        assert base.count(old) == 1, f"{name}: the mutated text occurs {base.count(old)} times in the oracle"
        jobs.append((name, base.replace(old, new)))
    workers = max(1, min(8, os.cpu_count() or 1))
    with cf.ThreadPoolExecutor(workers) as pool:
        results = list(pool.map(lambda j: _build_and_pin(str(tmp_path), *j), jobs))
    control = results[0]
    assert control[1] == 0, f"the unmutated oracle fails its pins under this harness:\n{control[2]}"
    survivors = [(n, out) for n, rc, out in results[1:] if rc == 0]
    broken = [(n, rc, out) for n, rc, out in results[1:] if rc not in (0, 1)]
    assert not broken, "mutants whose pin run did not end in a test failure:\n" + "\n".join(
        f"{n}: exit {rc}\n{out}" for n, rc, out in broken)
    assert not survivors, "mutants that pass every pin: " + ", ".join(n for n, _ in survivors)
