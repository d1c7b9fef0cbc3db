/* fp8_quotient.h -- the fp32 quotient y / sc used by the FP8 quantizer.
 *
 * q0 = y * inv is within about an ulp of y / sc when inv is the correctly
 * rounded 1 / sc; one Markstein correction step (the residual e = sc*q0 - y is
 * exact through the fused multiply-add) then yields the correctly rounded
 * quotient.  The residual is formed as sc*q0 - y and subtracted so that
 * y = -0 keeps its sign.  Plain C so the test suite can run it on the host
 * over every bf16 significand and every fp32 significand of sc. */
#ifndef RQ_FP8_QUOTIENT_H
#define RQ_FP8_QUOTIENT_H

#ifndef RQ_QUOTIENT_QUALIFIERS
#define RQ_QUOTIENT_QUALIFIERS static inline
#endif

RQ_QUOTIENT_QUALIFIERS float rq_fp8_quotient(float y, float sc, float inv) {
  float q0 = y * inv;
  float e = __builtin_fmaf(sc, q0, -y);
  return __builtin_fmaf(-e, inv, q0);
}

/* The FP8 scale amax / 448 for a bf16 amax: the same correction step with the
 * correctly rounded constant 1/448, exact for every bf16 amax in the normal
 * range. */
#define RQ_INV_448 (1.0f / 448.0f)
RQ_QUOTIENT_QUALIFIERS float rq_fp8_scale(float amax) { return rq_fp8_quotient(amax, 448.0f, RQ_INV_448); }

/* One Newton step on an approximate reciprocal r0 of sc.  For the scales that
 * occur (sc = amax / 448 rounded, amax a bf16 value: 128 significands) it
 * returns the correctly rounded 1 / sc from any r0 within 2 ulp of it; the
 * test suite checks every one of those significands and every such start. */
RQ_QUOTIENT_QUALIFIERS float rq_recip_refine(float sc, float r0) {
  float e = __builtin_fmaf(-sc, r0, 1.0f);
  return __builtin_fmaf(e, r0, r0);
}

#endif /* RQ_FP8_QUOTIENT_H */
