"""The kernels' division by launch-invariant divisors (``FastDiv`` in
rcc_internal.h: Granlund and Montgomery's multiply-high, add and shift) is
exact for every dividend below 2^31.

A host program compiled by hipcc includes the library's own header and
compares ``fdiv`` with the C++ ``/`` operator: every dividend up to 2^16 for
every divisor up to 256, and the edges (0, d - 1, d, d + 1, multiples of d
around 2^31, 2^31 - 1) plus pseudo-random dividends for divisors around
every power of two and pseudo-random divisors up to 2^31 - 1.  CPU only (the
program runs no GPU code).
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

PROGRAM = r"""
#include <stdio.h>
#include <stdint.h>
#include "rcc_internal.h"

static uint64_t state = 0x9E3779B97F4A7C15ull;
static uint32_t next31() {                 // xorshift64*, 31-bit outputs
  state ^= state >> 12; state ^= state << 25; state ^= state >> 27;
  return (uint32_t)((state * 0x2545F4914F6CDD1Dull) >> 33);
}

static long long bad = 0, checked = 0;
static void check(uint32_t n, uint32_t d, const rcc::FastDiv& f) {
  ++checked;
  if (rcc::fdiv(n, f) != n / d) {
    if (bad < 5) printf("mismatch n=%u d=%u got=%u want=%u\n", n, d, rcc::fdiv(n, f), n / d);
    ++bad;
  }
}
static void edges(uint32_t d) {
  const rcc::FastDiv f = rcc::make_fastdiv(d);
  const uint32_t top = 0x7fffffffu;
  const uint32_t cand[] = {0u, 1u, d - 1, d, d + 1, 2 * d - 1, top, top - 1,
                           (top / d) * d, (top / d) * d - 1, (top / d) * d + (d - 1 < top % d ? d - 1 : top % d)};
  for (uint32_t n : cand)
    if (n <= top) check(n, d, f);
  for (int i = 0; i < 200; ++i) check(next31(), d, f);
}

int main() {
  for (uint32_t d = 1; d <= 256; ++d) {
    const rcc::FastDiv f = rcc::make_fastdiv(d);
    for (uint32_t n = 0; n <= 65536; ++n) check(n, d, f);
    edges(d);
  }
  for (int k = 1; k < 31; ++k) {
    const uint32_t p = 1u << k;
    edges(p - 1);
    edges(p);
    edges(p + 1);
  }
  edges(0x7fffffffu);
  for (int i = 0; i < 20000; ++i) {
    const uint32_t d = next31();
    if (d) edges(d);
  }
  printf("%lld %lld\n", checked, bad);
  return bad != 0;
}
"""


def test_fastdiv_is_exact_below_2_pow_31():
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc missing")
    work = os.path.join(ROOT, "rope_chunk_causal_amd", "_build", "fastdiv_test")
    os.makedirs(work, exist_ok=True)
    src, exe = os.path.join(work, "fastdiv.cpp"), os.path.join(work, "fastdiv")
    with open(src, "w") as f:
        f.write(PROGRAM)
    r = subprocess.run([hipcc, "-x", "hip", "--offload-arch=gfx950", "-O2",
                        "-I", os.path.join(ROOT, "rope_chunk_causal_amd", "csrc"),
                        "-I", os.path.join(ROOT, "include"), src, "-o", exe],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr
    out = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    assert out.returncode == 0, out.stdout + out.stderr
    checked, bad = map(int, out.stdout.split()[-2:])
    assert bad == 0 and checked > 16_000_000
