"""The library's division by launch-invariant divisors (CPU only).

Several kernels split an index n < 2^31 by a divisor fixed for the launch (the
backward's row ids by k-1 and by G, the route's entry indices by G(k-1) and by
k-1) with FastDiv: a multiply-high, an add and a shift whose constants the host
builds (make_fastdiv). This compiles a host program against the library's own
header and compares fdiv(n, make_fastdiv(d)) with n / d for every divisor from 1
to 4096 at the boundaries where a rounding error would show first (each side of
the multiples of d near 0 and near 2^31, and 2^31 - 1) and at 20,000 random n per
divisor, and for d = 3, 7 and 12 at every n below 2^31.
"""
import os
import subprocess

import pytest

from block_sparse_attention_causal_amd import build as hip_build

CSRC = os.path.join(os.path.dirname(hip_build.__file__), "csrc")

PROGRAM = r"""
#include "moba_device.h"
#include <cstdio>
#include <cstdint>

static uint64_t state = 0x9E3779B97F4A7C15ull;
static uint32_t next31() {                 // xorshift64*, top 31 bits
  state ^= state >> 12; state ^= state << 25; state ^= state >> 27;
  return (uint32_t)((state * 0x2545F4914F6CDD1Dull) >> 33);
}

static long bad = 0, checked = 0;
static void check(uint32_t n, uint32_t d, moba::FastDiv f) {
  ++checked;
  if (moba::fdiv(n, f) != n / d) {
    if (bad < 10) printf("MISMATCH n=%u d=%u got=%u want=%u\n", n, d, moba::fdiv(n, f), n / d);
    ++bad;
  }
}

int main() {
  const uint32_t top = 0x7FFFFFFFu;
  for (uint32_t d = 1; d <= 4096; ++d) {
    const moba::FastDiv f = moba::make_fastdiv(d);
    for (uint32_t n = 0; n < 4 * d + 64; ++n) check(n, d, f);
    for (uint32_t k = top / d; k + 4 >= top / d && k > 0; --k)
      for (int o = -1; o <= 1; ++o) {
        const int64_t n = (int64_t)k * d + o;
        if (n >= 0 && n <= (int64_t)top) check((uint32_t)n, d, f);
      }
    check(top, d, f);
    for (int r = 0; r < 20000; ++r) check(next31(), d, f);
  }
  const uint32_t full[3] = {3, 7, 12};
  for (uint32_t d : full) {
    const moba::FastDiv f = moba::make_fastdiv(d);
    for (uint32_t n = 0; n <= top; ++n) {
      if (moba::fdiv(n, f) != n / d) { ++bad; break; }
      if (n == top) break;
    }
    checked += (long)top + 1;
  }
  printf("checked %ld bad %ld\n", checked, bad);
  return bad != 0;
}
"""


def test_fastdiv_matches_integer_division(tmp_path):
    src = tmp_path / "fastdiv_check.hip"
    src.write_text(PROGRAM)
    exe = str(tmp_path / "fastdiv_check")
    cmd = [hip_build.HIPCC, "-O2", "-std=c++17", "--offload-arch=" + hip_build.ARCH,
           "-I" + CSRC, "-I" + os.path.join(CSRC, "..", "..", "include"), str(src), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    r = subprocess.run([exe], capture_output=True, text=True, timeout=600)
    print(r.stdout)
    assert r.returncode == 0, r.stdout[-2000:]
    assert "bad 0" in r.stdout
