"""The encoders' division x / d: computed as q = x r with r = RN(1 / d), then
two residual corrections q += fma(-d, q, x) r and the sign of x.  This host
test restates that sequence in C (glibc's fmaf is correctly rounded) and
checks it against IEEE division over every finite BF16 dividend and a spread
of divisors in [2^-64, 2^64] (the range the kernels take it in), plus random
dividends placed within a few ulps of quotients of every magnitude.  Results
may differ only below 2^-40, where every code of both formats is zero."""
import os
import shutil
import subprocess

import pytest

SRC = r"""
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>
static float f(uint32_t b) { float x; memcpy(&x, &b, 4); return x; }
static uint32_t bits(float x) { uint32_t b; memcpy(&b, &x, 4); return b; }
static float div_rn(float x, float d, float r) {
  float q = x * r;
  q = fmaf(fmaf(-d, q, x), r, q);
  q = fmaf(fmaf(-d, q, x), r, q);
  return copysignf(q, x);
}
static uint64_t s = 88172645463325252ull;
static uint64_t rnd(void) { s ^= s << 13; s ^= s >> 7; s ^= s << 17; return s; }
static float sig(void) { return 1.0f + (float)(rnd() & 0x7FFFFF) / 8388608.0f; }
int main(void) {
  long long n = 0, bad = 0;
  const float lim = ldexpf(1.0f, 64), tiny = ldexpf(1.0f, -40);
  for (int trial = 0; trial < 600; ++trial) {
    int e = (int)(rnd() % 129) - 64;
    float d = ldexpf(sig(), e);
    if (trial % 7 == 0) d = ldexpf(1.0f, e);
    if (trial % 11 == 0) d = ldexpf(1.99999988f, e);
    if (trial < 126) d = f(0x3F800000u + ((uint32_t)trial << 17)) * 0.7654321f;
    const float r = 1.0f / d;
    for (uint32_t hb = 0; hb < 65536; ++hb) {
      const float x = f(hb << 16);
      if (!isfinite(x)) continue;
      const float q = x / d;
      if (fabsf(q) > lim) continue;
      const float g = div_rn(x, d, r);
      ++n;
      if (bits(g) != bits(q) && (fabsf(q) >= tiny || fabsf(g) >= 2 * tiny)) {
        if (bad < 5) printf("x=%a d=%a q=%a got=%a\n", x, d, q, g);
        ++bad;
      }
    }
  }
  for (long long i = 0; i < 20000000ll; ++i) {
    float d = ldexpf(sig(), (int)(rnd() % 129) - 64);
    float r = 1.0f / d;
    float x = ldexpf(sig(), (int)(rnd() % 60) - 40) * d;
    x = f(bits(x) + (uint32_t)(rnd() % 9) - 4);
    if (rnd() & 1) x = -x;
    if (!isfinite(x)) continue;
    float q = x / d, g = div_rn(x, d, r);
    ++n;
    if (bits(g) != bits(q) && (fabsf(q) >= tiny || fabsf(g) >= 2 * tiny)) {
      if (bad < 5) printf("x=%a d=%a q=%a got=%a\n", x, d, q, g);
      ++bad;
    }
  }
  printf("checked %lld mismatches %lld\n", n, bad);
  return bad != 0;
}
"""


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_division_sequence_is_ieee_division(tmp_path):
    c = tmp_path / "div_rn.c"
    c.write_text(SRC)
    exe = tmp_path / "div_rn"
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", str(c), "-o", str(exe), "-lm"], check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300)
    assert out.returncode == 0, out.stdout
    assert "mismatches 0" in out.stdout
