"""The RMSNorm kernel forms fl(x / r) without the division sequence: with
y = fl(1 / r) (correctly rounded) and q0 = fl(x * y), the quotient is
fl(q0 + fl(x - q0 * r) * y) computed with two fused multiply-adds, which is
Markstein's theorem on division by a correctly rounded reciprocal; the
kernel divides as written when |x| or |q0| lies outside [2^-80, 2^100].
This checks the identity, with that guard, against IEEE division on the
CPU (C's fmaf and '/'), over random fp32 pairs and over quotients next to
ties (x one ulp either side of fl(q * r)).  CPU only."""
import os
import subprocess

import pytest

SRC = r"""
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>
static float f_of(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t u_of(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
static uint64_t st = 0x9E3779B97F4A7C15ull;
static uint64_t rnd(void) { st ^= st << 13; st ^= st >> 7; st ^= st << 17; return st; }
static float quotient(float x, float r, float y) {
  float q0 = x * y, aq = fabsf(q0);
  if (fabsf(x) >= 0x1p-80f && aq >= 0x1p-80f && aq <= 0x1p100f)
    return fmaf(fmaf(-q0, r, x), y, q0);
  return x == 0.0f ? q0 : x / r;
}
static long bad = 0, n = 0;
static void check(float x, float r, float y) {
  float want = x / r, got = quotient(x, r, y);
  ++n;
  if (u_of(got) != u_of(want) && !(got == 0.0f && want == 0.0f)) {
    if (bad < 5) printf("mismatch r=%a x=%a want=%a got=%a\n", r, x, want, got);
    ++bad;
  }
}
int main(void) {
  float rs[40] = {1.0f, 3.0f, 0.1f, 0.0031622776f, 1.0000001f, 0.99999994f, 0x1p-8f, 7.0f};
  int nr = 8;
  while (nr < 40) {
    float r = f_of((uint32_t)(rnd() % (254u << 23)) + (1u << 23));
    if (isfinite(r) && r > 0x1p-9f && r < 0x1p70f) rs[nr++] = r;
  }
  for (int i = 0; i < nr; ++i) {
    const float r = rs[i], y = 1.0f / r;
    for (long k = 0; k < (1L << 18); ++k) {
      float x = f_of((uint32_t)rnd());
      if (isfinite(x)) check(x, r, y);
    }
    for (long k = 0; k < (1L << 16); ++k) {
      float q = f_of(0x3f800000u + (uint32_t)(rnd() % (1u << 23)));
      float x = q * r;
      check(x, r, y);
      check(nextafterf(x, INFINITY), r, y);
      check(nextafterf(x, -INFINITY), r, y);
    }
  }
  printf("checked %ld mismatches %ld\n", n, bad);
  return bad != 0;
}
"""


def test_corrected_reciprocal_quotient_is_ieee_division(tmp_path):
    src = tmp_path / "div.c"
    exe = tmp_path / "div"
    src.write_text(SRC)
    try:
        subprocess.run(["gcc", "-O2", "-ffp-contract=off", str(src), "-o", str(exe), "-lm"],
                       check=True, capture_output=True)
    except (OSError, subprocess.CalledProcessError) as e:
        pytest.skip("no C compiler: %r" % (e,))
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "mismatches 0" in r.stdout
