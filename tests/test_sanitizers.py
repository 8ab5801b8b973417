"""AddressSanitizer + UndefinedBehaviorSanitizer on the CPU code (no GPU).

Two sanitized builds, each loaded in a subprocess of its own (each carries
its compiler's sanitizer runtime, preloaded):
  * the oracle (g++ -fsanitize=address,undefined), under the oracle's pin
    tests;
  * the library with its host code sanitized (hipcc with every -fsanitize=
    behind -Xarch_host: the gfx950 device code is built as usual and never
    runs here), under the C ABI and binding tests, which exercise the
    argument validation and error paths of every entry point.
Any report aborts the subprocess (halt_on_error / abort_on_error), which
fails the test.  Leak checking is off: the Python interpreter and torch keep
allocations alive until exit by design.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from bit_w4a4_quantized_smooth_amd import build as pkg_build  # noqa: E402
from oracle import build as oracle_build  # noqa: E402

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}

# confirms, inside the subprocess, that the sanitized library and a sanitizer
# runtime are the ones mapped
PROBE = """
import sys
sys.path.insert(0, {root!r})
{load}
maps = open('/proc/self/maps').read()
assert {lib!r} in maps, 'sanitized library not loaded'
assert 'asan' in maps, 'no sanitizer runtime mapped'
print('sanitized build mapped')
"""


def _run(env_extra, args, timeout):
    env = dict(os.environ)
    env.update(SAN_ENV)
    env.update(env_extra)
    return subprocess.run([sys.executable] + args, cwd=ROOT, env=env, capture_output=True, text=True,
                          timeout=timeout)


def _check(r):
    assert r.returncode == 0, f"exit {r.returncode}\n{r.stdout[-4000:]}\n{r.stderr[-4000:]}"


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not found")
def test_oracle_under_asan_ubsan(tmp_path):
    lib = str(tmp_path / "liboracle_san.so")
    subprocess.run(["g++", "-O1", "-g", "-std=c++17", "-ffp-contract=off", "-fno-fast-math", "-shared", "-fPIC",
                    "-pthread", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                    "-fno-omit-frame-pointer", oracle_build.SRC, "-o", lib], check=True, timeout=300)
    runtime = subprocess.run(["g++", "-print-file-name=libasan.so"], capture_output=True, text=True,
                             check=True).stdout.strip()
    env = {"SVDQ_ORACLE_LIB": lib, "LD_PRELOAD": runtime}
    _check(_run(env, ["-c", PROBE.format(root=ROOT, load="import oracle; oracle._lib()", lib=lib)], 120))
    tests = [os.path.join(ROOT, "tests", t) for t in
             ("test_oracle_converters.py", "test_oracle_method.py", "test_oracle_mlp.py", "test_oracle_qkv.py",
              "test_oracle_offline.py")]
    r = _run(env, ["-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu"] + tests, 900)
    print(r.stdout[-600:])
    _check(r)


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not found")
def test_host_layer_under_asan_ubsan(tmp_path):
    lib = str(tmp_path / "libsvdq_san.so")
    flags = [f for f in pkg_build.HIPCC_FLAGS if f != "-O3"] + [
        "-O1", "-g",
        "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
        "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
    subprocess.run([HIPCC] + flags + [os.path.join(pkg_build.CSRC, s) for s in pkg_build.SOURCES] + ["-o", lib],
                   check=True, timeout=900, capture_output=True)
    clang = os.path.join(os.path.dirname(os.path.realpath(HIPCC)), "..", "llvm", "bin", "clang")
    if not os.path.exists(clang):
        clang = "/opt/rocm/llvm/bin/clang"
    runtime = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True,
                             text=True, check=True).stdout.strip()
    if not os.path.isabs(runtime) or not os.path.exists(runtime):
        import glob
        found = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
        assert found, "clang's AddressSanitizer runtime not found"
        runtime = found[0]
    env = {"SVDQ_LIB": lib, "LD_PRELOAD": runtime}
    _check(_run(env, ["-c", PROBE.format(root=ROOT, load="import bit_w4a4_quantized_smooth_amd as sq; sq.lib()",
                                         lib=lib)], 120))
    tests = [os.path.join(ROOT, "tests", t) for t in ("test_abi.py", "test_binding.py")]
    r = _run(env, ["-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu"] + tests, 900)
    print(r.stdout[-600:])
    _check(r)
