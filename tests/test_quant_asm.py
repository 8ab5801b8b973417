"""The quantizer's ring waits count memory instructions by hand: round j waits
until at most a fixed number of vector-memory operations issued after its own
copies are still in flight.  That is only right if the compiler emits the
prologue's operations as written: three rounds of copies (buffer loads to
LDS), each followed by its pair of dropped stores.  Identical dropped stores
were once merged into one pair by the compiler, which left round 0's wait
short of round 0's copies (the first round then read X slices before they
landed).  This test builds quant_act.hip for gfx950 with the library's flags
and checks, in the assembly of every LDS-staged quantizer kernel and every
fused quantizer + GEMV kernel, that before the first barrier

  * every round's copies are followed by its two stores (three pairs), and
  * the wait in front of that barrier leaves in flight no more operations
    than were issued after round 0's copies;

and that every later round (barrier to barrier) issues its copies (one more
where the next reciprocal chunk is copied) and then exactly its two stores.

CPU only (the compiler runs here; nothing is launched)."""
import os
import re
import subprocess
import tempfile

import pytest

from bit_w4a4_quantized_smooth_amd import build as pkg_build

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SRC = os.path.join(pkg_build.CSRC, "quant_act.hip")


@pytest.fixture(scope="module")
def asm():
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    flags = [f for f in pkg_build.HIPCC_FLAGS if f not in ("-shared", "-fPIC")]
    with tempfile.TemporaryDirectory() as d:
        out = os.path.join(d, "quant_act.s")
        subprocess.run([HIPCC] + flags + ["--offload-device-only", "-S", SRC, "-o", out], check=True,
                       stderr=subprocess.DEVNULL)
        return open(out).read()


def prologue(body):
    """Memory operations from the first copy to LDS up to the first barrier:
    'C' copy, 'S' store, 'L' register load, ('W', n) a vmcnt(n) wait."""
    seq = []
    started = False
    for line in body:
        t = line.strip()
        if not started:
            started = t.startswith("buffer_load") and " lds" in t
            if not started:
                continue
        if t.startswith("s_barrier"):
            return seq
        if t.startswith("buffer_load"):
            seq.append("C" if " lds" in t else "L")
        elif t.startswith(("buffer_store", "global_store")):
            seq.append("S")
        elif t.startswith("s_waitcnt") and "vmcnt" in t:
            seq.append(("W", int(re.search(r"vmcnt\((\d+)\)", t).group(1))))
    raise AssertionError("no barrier after the prologue")


def test_ring_prologue_order(asm):
    names = re.findall(r"^(_ZN4svdq(?:20quant_act_dma_kernel|16quant_awq_kernel)\S+):", asm, re.M)
    assert len(names) >= 16, "quantizer kernels not found in the assembly"
    for name in names:
        i = asm.index(name + ":")
        body = asm[i:asm.index(".Lfunc_end", i)].split("\n")
        seq = prologue(body)
        ops = [x for x in seq if not isinstance(x, tuple)]
        ndma = ops.index("S")  # copies of round 0
        assert ndma >= 3, (name, ops)
        rounds = "".join(x for x in ops if x in "CS")
        assert rounds.startswith(("C" * ndma + "SS") * 3), (name, rounds)
        after0 = len(ops) - ndma  # operations issued after round 0's copies
        waits = [x[1] for x in seq if isinstance(x, tuple)]
        assert waits and waits[-1] <= after0, (name, "round 0 wait", waits[-1], "after", after0)


def test_ring_rounds_order(asm):
    names = re.findall(r"^(_ZN4svdq(?:20quant_act_dma_kernel|16quant_awq_kernel)\S+):", asm, re.M)
    for name in names:
        i = asm.index(name + ":")
        body = asm[i:asm.index(".Lfunc_end", i)].split("\n")
        ndma = [x for x in prologue(body) if not isinstance(x, tuple)].index("S")
        blocks, cur, seen = [], [], False
        for line in body:
            t = line.strip()
            if t.startswith("buffer_load") and " lds" in t:
                seen = True
                cur.append("C")
            elif t.startswith("buffer_store") and seen:
                cur.append("S")
            elif t.startswith("s_barrier") and seen:
                blocks.append("".join(cur))
                cur = []
        rounds = [b for b in blocks[1:] if "C" in b]  # after the prologue, up to the epilogue
        assert rounds, name
        ok = {"C" * ndma + "SS", "C" * (ndma + 1) + "SS"}
        assert all(b in ok for b in rounds), (name, sorted(set(rounds)))
