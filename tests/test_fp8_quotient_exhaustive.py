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

import pytest

PKG = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "rmsnorm_activation_quantization_amd", "csrc")

PROGRAM_TEMPLATE = r"""
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
    for (int m = 0; m < (1 << FRAC_BITS); ++m) {
      uint32_t yu = 0x3F800000u | ((uint32_t)m << (23 - FRAC_BITS));  /* significand of the element type */
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


@pytest.mark.parametrize("frac_bits", [7, 10], ids=["bf16", "fp16"])
def test_quotient_is_correctly_rounded(tmp_path, frac_bits):
    """Every significand of the element type (bf16: 7 fraction bits, fp16: 10)
    against every fp32 divisor significand."""
    src = tmp_path / "quotient_check.c"
    src.write_text(f"#define FRAC_BITS {frac_bits}\n" + PROGRAM_TEMPLATE)
    exe = tmp_path / "quotient_check"
    subprocess.run(["gcc", "-O2", "-mfma", "-ffp-contract=off", "-fopenmp", "-I", PKG, str(src), "-o", str(exe)],
                   check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=600)
    assert out.returncode == 0 and "mismatches 0" in out.stdout, out.stdout + out.stderr


SCALE_PROGRAM = r"""
#include <math.h>
#include <stdio.h>
#include <string.h>
#include <stdint.h>
#include "fp8_quotient.h"
static uint32_t bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
static float from(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
int main(void) {
  long long bad = 0;
  /* every bf16 amax from 2^-54 up to the largest finite bf16 (the kernel's fast
     path), then every positive finite fp16 amax */
  for (uint32_t n = 0; n < 0x7F80u - (73u << 7) + 0x7C00u; ++n) {
    float amax;
    if (n < 0x7F80u - (73u << 7)) {
      amax = from(((73u << 7) + n) << 16);
    } else {
      uint32_t hb = n - (0x7F80u - (73u << 7));      /* fp16 bits 0x0000..0x7BFF */
      uint32_t e = hb >> 10, m = hb & 0x3FFu;
      amax = e ? ldexpf(1.0f + (float)m / 1024.0f, (int)e - 15) : ldexpf((float)m, -24);
      if (amax == 0.0f) continue;
    }
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
    """Every bf16 amax on the fast path, and every fp16 amax: the division-free scale equals
    RN(amax / 448), and one Newton step from any estimate within 2 ulp gives
    RN(1 / scale) (the hardware reciprocal estimate is within 1 ulp)."""
    src = tmp_path / "scale_check.c"
    src.write_text(SCALE_PROGRAM)
    exe = tmp_path / "scale_check"
    subprocess.run(["gcc", "-O2", "-mfma", "-ffp-contract=off", "-I", PKG, str(src), "-o", str(exe), "-lm"], check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert out.returncode == 0 and "mismatches 0" in out.stdout, out.stdout + out.stderr
