"""Host check of the append kernel's division by multiplication (div_magic in
csrc/hn_internal.h): n / d == (n * m) >> k for numerators below 2^31.

A small host program includes the header, so the code under test is the
library's own; every quotient it computes is compared with Python's exact
integer division.  Divisors: 1..4096, every power of two and its neighbours
up to 2^31, and seeded random divisors; numerators: 0, d - 1, d, d + 1, the
largest multiple of d below 2^31 and its neighbours, 2^31 - 1 and seeded
random values."""
import os
import random
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"

PROGRAM = r"""
#include <cstdio>
#include "hn_internal.h"
int main() {
  unsigned long long d, n;
  while (std::scanf("%llu %llu", &d, &n) == 2) {
    uint32_t m; int32_t k;
    hn::div_magic((uint32_t)d, m, k);
    std::printf("%llu\n", (unsigned long long)(((uint64_t)n * m) >> k));
  }
  return 0;
}
"""


def cases():
    rng = random.Random(20261204)
    ds = list(range(1, 4097))
    for e in range(31):
        ds += [2 ** e - 1, 2 ** e, 2 ** e + 1]
    ds += [rng.randrange(1, 2 ** 31) for _ in range(2000)]
    top = 2 ** 31 - 1
    out = []
    for d in sorted(set(x for x in ds if 1 <= x < 2 ** 31)):
        mult = top // d * d
        ns = {0, d - 1, d, d + 1, mult, mult - 1, top, top - 1}
        ns |= {rng.randrange(0, 2 ** 31) for _ in range(8)}
        out += [(d, n) for n in ns if 0 <= n <= top]
    return out


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="needs hipcc to build the host program")
def test_div_magic_matches_integer_division(tmp_path):
    src = tmp_path / "dm.cpp"
    src.write_text(PROGRAM)
    exe = tmp_path / "dm"
    rocm_inc = os.path.join(os.path.dirname(os.path.dirname(os.path.realpath(HIPCC))), "include")
    r = subprocess.run([HIPCC, "-O2", "-std=c++17", "-x", "c++", "-D__HIP_PLATFORM_AMD__",
                        "-I", rocm_inc, "-I", os.path.join(ROOT, "include"),
                        "-I", os.path.join(ROOT, "masked_attention_hn_amd", "csrc"),
                        str(src), "-o", str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    cs = cases()
    inp = "".join(f"{d} {n}\n" for d, n in cs)
    r = subprocess.run([str(exe)], input=inp, capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    got = [int(x) for x in r.stdout.split()]
    assert len(got) == len(cs)
    bad = [(d, n, g) for (d, n), g in zip(cs, got) if g != n // d]
    assert not bad, bad[:10]
