"""Builds libsvdq.so (the gfx950 HIP kernels and their C ABI) in-tree.

Every HIP source is compiled for gfx950 only, with
  * matrix-core instructions in their VGPR form,
  * packed-fp32 instructions disabled (the compiler would otherwise form
    v_pk_*_f32 from plain float code),
  * IEEE-correct fp32 division and fp32 denormals kept, because the
    quantizer's decisions must match the oracle bit for bit.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libsvdq.so")
SOURCES = ["svdq_api.hip", "quant_act.hip", "gemm_int4.hip", "gemm_nvfp4.hip", "awq_gemv.hip", "offline.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fhip-fp32-correctly-rounded-divide-sqrt", "-fno-gpu-flush-denormals-to-zero",
    # matrix-core results land in VGPRs, where the vector ALU reads them
    # directly (the AGPR form would need a v_accvgpr_read per element)
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wall", "-Wno-unused-function",
]


def build(verbose: bool = False, extra_flags=None) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    out_tmp = LIB + ".tmp"
    cmd = [hipcc] + HIPCC_FLAGS + list(extra_flags or []) + srcs + ["-o", out_tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(out_tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True, extra_flags=sys.argv[1:]))
