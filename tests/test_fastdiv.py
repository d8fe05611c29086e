"""Host check of the launch-constant division (csrc/fastdiv.h): the kernels
divide row and unit indices by launch constants with one high multiply, an add
and a shift.  The constants and the formula are checked here against plain
integer division, exhaustively for small divisors and dividends and at the
ends of the dividend range [0, 2^31) for divisors up to 2^31 - 1."""
import os
import shutil
import subprocess
import tempfile

import pytest

CSRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "paged_quantized_kv_ra_amd", "csrc")

PROGRAM = r"""
#include <stdio.h>
#include <stdint.h>
#include <initializer_list>
#include "fastdiv.h"
static uint64_t state = 0x9E3779B97F4A7C15ull;
static uint32_t rnd() { state ^= state << 13; state ^= state >> 7; state ^= state << 17; return (uint32_t)state; }
static int check(uint32_t d, uint32_t n) {
  const ra::FastDiv f = ra::make_fastdiv(d);
  const uint32_t hi = (uint32_t)(((uint64_t)f.m * n) >> 32);
  const uint32_t q = ra::fastdiv_apply(f, hi, n);
  if (f.d != d || q != n / d) { printf("FAIL d=%u n=%u q=%u want %u\n", d, n, q, n / d); return 1; }
  return 0;
}
int main() {
  const uint32_t top = 0x7FFFFFFFu;
  for (uint32_t d = 1; d <= 1024; ++d) {
    for (uint32_t n = 0; n < 70000; ++n) if (check(d, n)) return 1;
    for (uint32_t n = top - 70000; n < top; ++n) if (check(d, n)) return 1;
    if (check(d, top)) return 1;
  }
  for (int i = 0; i < 2000000; ++i) {
    uint32_t d = 1 + rnd() % top, n = rnd() & top;
    if (check(d, n) || check(d, top) || check(d, d) || check(d, d - 1)) return 1;
  }
  for (uint32_t e = 0; e < 31; ++e) {
    const uint32_t p = 1u << e;
    for (uint32_t d : {p, p + 1, p > 1 ? p - 1 : 1u})
      for (uint32_t n : {0u, 1u, d - 1, d, d + 1, 2 * d - 1, top / d * d - 1, top / d * d, top})
        if (n <= top && check(d, n)) return 1;
  }
  printf("OK\n");
  return 0;
}
"""


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_fastdiv_matches_integer_division():
    with tempfile.TemporaryDirectory() as d:
        src = os.path.join(d, "t.cpp")
        exe = os.path.join(d, "t")
        with open(src, "w") as f:
            f.write(PROGRAM)
        subprocess.run(["g++", "-O2", "-std=c++17", "-I", CSRC, src, "-o", exe], check=True)
        r = subprocess.run([exe], capture_output=True, text=True, timeout=300)
        assert r.returncode == 0 and r.stdout.strip() == "OK", r.stdout + r.stderr
