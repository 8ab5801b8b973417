"""The int4 activation quantizer computes the group scale fl32(amax / 7) without
a division: q0 = fl32(a * fl32(1/7)), r = fma(-q0, 7, a), q1 = fma(r, fl32(1/7), q0)
(csrc/common.h, div7_rn).  This test checks that identity exhaustively on the
CPU: for every non-negative finite float a (2^31 - 2^23 values, subnormals
included), q1 equals the IEEE-rounded quotient a / 7.  The same two IEEE
operations (a float multiply and a fused multiply-add) run on the GPU's vector
ALU, so the sequence gives the scale bit for bit there too."""
import os
import subprocess
import tempfile

SRC = r"""
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>
#define NTHREADS 8
static const uint32_t END = 0x7F800000u;  /* +inf: every finite non-negative float below it */
static unsigned long long bad[NTHREADS];
static void* run(void* arg) {
  const int id = (int)(intptr_t)arg;
  const float r7 = 1.0f / 7.0f;
  const uint32_t lo = (uint32_t)((uint64_t)END * id / NTHREADS), hi = (uint32_t)((uint64_t)END * (id + 1) / NTHREADS);
  for (uint32_t b = lo; b < hi; ++b) {
    float a; memcpy(&a, &b, 4);
    volatile float want = a / 7.0f;
    const float q0 = a * r7;
    const float r = fmaf(-q0, 7.0f, a);
    const float q1 = fmaf(r, r7, q0);
    uint32_t x, y; float w = want; memcpy(&x, &q1, 4); memcpy(&y, &w, 4);
    if (x != y) ++bad[id];
  }
  return 0;
}
int main(void) {
  pthread_t t[NTHREADS];
  for (int i = 0; i < NTHREADS; ++i) pthread_create(&t[i], 0, run, (void*)(intptr_t)i);
  unsigned long long total = 0;
  for (int i = 0; i < NTHREADS; ++i) { pthread_join(t[i], 0); total += bad[i]; }
  printf("%llu\n", total);
  return 0;
}
"""


def test_div7_matches_ieee_division_for_all_nonnegative_floats():
    with tempfile.TemporaryDirectory() as d:
        src, exe = os.path.join(d, "div7.c"), os.path.join(d, "div7")
        open(src, "w").write(SRC)
        subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-pthread", src, "-o", exe, "-lm"],
                       check=True)
        out = subprocess.run([exe], check=True, capture_output=True, text=True, timeout=600).stdout
    assert int(out.strip()) == 0, f"{out.strip()} mismatches"
