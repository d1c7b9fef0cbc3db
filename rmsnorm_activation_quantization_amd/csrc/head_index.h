/* head_index.h -- token and head of a flat head index u = token * d + head.
 *
 * The QK kernel numbers the heads of a launch 0, 1, 2, ... across tokens, with
 * d = Hq + Hk heads a token and u < 2^31.  A division by the launch-invariant d
 * is replaced by a multiply and a shift (Granlund and Montgomery, "Division by
 * invariant integers using multiplication", PLDI 1994): with l = ceil(log2 d)
 * and m = ceil(2^(31+l) / d), floor(u / d) = floor(u * m / 2^(31+l)) for every
 * 0 <= u < 2^31, because 2^(31+l) <= m * d < 2^(31+l) + d <= 2^(31+l) + 2^l.
 * m < 2^32 for every d >= 1, and u * m < 2^63.  Plain C so the test suite can
 * check it on the host for every d up to 2^17. */
#ifndef RQ_HEAD_INDEX_H
#define RQ_HEAD_INDEX_H

#include <stdint.h>

#ifndef RQ_HEAD_INDEX_QUALIFIERS
#define RQ_HEAD_INDEX_QUALIFIERS static inline
#endif

typedef struct rq_head_divisor {
  uint32_t magic;  /* m */
  uint32_t shift;  /* 31 + l */
} rq_head_divisor;

/* For 1 <= d <= 2^31. */
static inline rq_head_divisor rq_head_divisor_of(uint32_t d) {
  uint32_t l = 0;
  while (((uint64_t)1 << l) < d) ++l;
  const uint64_t p = (uint64_t)1 << (31 + l);
  rq_head_divisor r;
  r.magic = (uint32_t)((p + d - 1) / d);
  r.shift = 31 + l;
  return r;
}

/* floor(u / d) for u < 2^31. */
RQ_HEAD_INDEX_QUALIFIERS uint32_t rq_head_quotient(uint32_t u, uint32_t magic, uint32_t shift) {
  return (uint32_t)(((uint64_t)u * magic) >> shift);
}

#endif
