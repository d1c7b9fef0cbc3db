"""Host check of the FP8 quantizer's quotient step (csrc/fp8_quotient.h).

The kernel forms y / scale as a reciprocal multiply plus one Markstein
correction.  Binary floating-point division is invariant under power-of-two
scaling of either operand (away from underflow and overflow), so running every
bf16 significand of y (128) against every fp32 significand of the divisor
(2^23) covers every case the kernel meets with scale >= 2^-64.  Each result must
equal the IEEE fp32 quotient, obtained here as the double quotient rounded to
fp32 (53 >= 2*24 + 2 bits, so that double rounding is innocuous).
Signed zeros are checked on the GPU through the kernel itself (the host
compiler's optimizer does not keep the sign of a zero fma result)."""

import os
import subprocess

PKG = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "rmsnorm_activation_quantization_amd", "csrc")

PROGRAM = r"""
#include <stdio.h>
#include <string.h>
#include <stdint.h>
#include "fp8_quotient.h"
static uint32_t bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
int main(void) {
  long long bad = 0;
  #pragma omp parallel for reduction(+:bad) schedule(static)
  for (int k = 0; k < (1 << 23); ++k) {
    uint32_t su = 0x3F800000u | (uint32_t)k;   /* divisor in [1, 2) */
    float sc; memcpy(&sc, &su, 4);
    float inv = 1.0f / sc;                      /* correctly rounded */
    for (int m = 0; m < 128; ++m) {
      uint32_t yu = 0x3F800000u | ((uint32_t)m << 16);  /* bf16 significand in [1, 2) */
      float y; memcpy(&y, &yu, 4);
      float want = (float)((double)y / (double)sc);
      float got = rq_fp8_quotient(y, sc, inv);
      float gotn = rq_fp8_quotient(-y, sc, inv);
      if (bits(got) != bits(want) || bits(gotn) != bits(-want)) ++bad;
    }
  }
  /* an exact e4m3 midpoint: scale 3, y = 51/16 -> 1.0625 exactly */
  if (rq_fp8_quotient(3.1875f, 3.0f, 1.0f / 3.0f) != 1.0625f) ++bad;
  printf("mismatches %lld\n", bad);
  return bad != 0;
}
"""


def test_quotient_is_correctly_rounded(tmp_path):
    src = tmp_path / "quotient_check.c"
    src.write_text(PROGRAM)
    exe = tmp_path / "quotient_check"
    subprocess.run(["gcc", "-O2", "-mfma", "-ffp-contract=off", "-fopenmp", "-I", PKG, str(src), "-o", str(exe)],
                   check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=600)
    assert out.returncode == 0 and "mismatches 0" in out.stdout, out.stdout + out.stderr


SCALE_PROGRAM = r"""
#include <stdio.h>
#include <string.h>
#include <stdint.h>
#include "fp8_quotient.h"
static uint32_t bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
static float from(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
int main(void) {
  long long bad = 0;
  /* every bf16 amax from 2^-54 up to the largest finite bf16 (the kernel's fast path) */
  for (uint32_t ab = (73u << 7); ab < 0x7F80u; ++ab) {
    float amax = from(ab << 16);
    float want = (float)((double)amax / 448.0);          /* RN(amax / 448) */
    float scale = rq_fp8_scale(amax);
    if (bits(scale) != bits(want)) ++bad;
    float inv = (float)(1.0 / (double)want);              /* RN(1 / scale) */
    for (int d = -2; d <= 2; ++d)                          /* any hardware estimate within 2 ulp */
      if (bits(rq_recip_refine(want, from(bits(inv) + d))) != bits(inv)) ++bad;
  }
  printf("mismatches %lld\n", bad);
  return bad != 0;
}
"""


def test_scale_and_reciprocal_are_correctly_rounded(tmp_path):
    """Every bf16 amax on the fast path: the division-free scale equals
    RN(amax / 448), and one Newton step from any estimate within 2 ulp gives
    RN(1 / scale) (the hardware reciprocal estimate is within 1 ulp)."""
    src = tmp_path / "scale_check.c"
    src.write_text(SCALE_PROGRAM)
    exe = tmp_path / "scale_check"
    subprocess.run(["gcc", "-O2", "-mfma", "-ffp-contract=off", "-I", PKG, str(src), "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert out.returncode == 0 and "mismatches 0" in out.stdout, out.stdout + out.stderr
