// rq_oracle.cpp -- plain, slow, obviously correct CPU oracle.
//
// TEST INFRASTRUCTURE ONLY: the checker for the HIP library.  Loaded only by
// the tests, the smoke check and the benchmark's CPU-baseline leg.  It shares
// no code with the HIP library and is built by g++ from this file alone.
//
// Precision: every real-valued intermediate is a double; the only roundings
// are the ones the definition names (bf16 at each tensor boundary, fp32 for the
// FP8 scale and quotient, the target code format).  No blocking, no fusion, no
// reordering: one row at a time, one element at a time, in index order.
//
// Page citations (by page and section):
//   [P1] sglang PR #29723 -- fused AllReduce + RMSNorm + quant (per-token FP8,
//        MXFP4) on AMD.  Motivation: the unfused sequence is
//        residual add -> RMSNorm -> quantize with bf16 round trips between the
//        launches.  Accuracy Tests: the fused kernel is numerically equivalent
//        to that sequence.  Key changes: output tuple (codes, residual_out,
//        per-token scale (M, 1)).  Review notes: optional bf16 side output.
//   [P2] sgl-amd-mono PR #26 "[Feat] [MI355X] muse_spark: Whole-layer
//        monokernels for Muse Spark", commit notes: the MXFP4 blocks are the
//        quantization of the bf16 normalized row.
//   [P4] sglang PR #27656 "[AMD][Perf] Fuse QK RMSNorm + gate extraction
//        Triton kernel for Qwen3.5 on HIP", Motivation and Modifications.
// The pages leave the formulas open; the workload statement fixes
// scale = amax / 448 for FP8 and the E8M0 exponent floor(log2 amax) - 2 with
// one scale per 32 elements for MXFP4.  Readings of silent points:
//   - the norm reads the bf16-rounded residual_out (the unfused sequence
//     stores it as bf16 before the norm kernel reads it) [P1 Motivation];
//   - mean of squares divides by H; eps is added inside the square root;
//   - the normalized row is rounded once to bf16 and the quantizer reads that
//     bf16 row [P1 Motivation, P2 commit notes];
//   - FP8 is OCP E4M3FN (max 448), nearest-even, saturating; the quotient
//     y / scale is an IEEE fp32 division, like the scale itself;
//   - an all-zero granule has scale 0 (FP8) or E8M0 byte 0 and codes that
//     keep only the sign of zero;
//   - E2M1 rounds to nearest-even on {0, .5, 1, 1.5, 2, 3, 4, 6}, saturating;
//     element 2j goes in the low nibble of byte j;
//   - GemmaRMSNorm multiplies by (1 + w) [P4 Modifications].

#include "rq_oracle.h"

#include <cmath>
#include <cstring>
#include <vector>

namespace {

double bf16_value(uint16_t b) {
  // A bf16 is the upper half of an IEEE binary32.
  uint32_t u = (uint32_t)b << 16;
  float f;
  std::memcpy(&f, &u, sizeof f);
  return (double)f;
}

uint16_t bf16_round(double v) {
  const uint16_t sign = std::signbit(v) ? 0x8000 : 0;
  if (std::isnan(v)) return (uint16_t)(sign | 0x7FC0);
  double a = std::fabs(v);
  if (a == 0.0) return sign;
  if (std::isinf(a)) return (uint16_t)(sign | 0x7F80);
  // bf16 keeps 8 significant bits; normal exponents -126..127, and below
  // 2^-126 the spacing stays 2^-133 (subnormals).
  int e = std::ilogb(a);
  int quantum_exp = (e < -126) ? -133 : e - 7;
  double n = std::nearbyint(std::ldexp(a, -quantum_exp));  // ties to even
  double r = std::ldexp(n, quantum_exp);
  if (r > 0x1.FEp127) return (uint16_t)(sign | 0x7F80);  // rounds past the largest finite bf16
  float f = (float)r;  // exact: r is a bf16 value
  uint32_t u;
  std::memcpy(&u, &f, sizeof u);
  return (uint16_t)(sign | (u >> 16));
}

double f16_value(uint16_t b) {
  // IEEE binary16: sign, 5 exponent bits (bias 15), 10 mantissa bits.
  const double s = (b & 0x8000) ? -1.0 : 1.0;
  const int e = (b >> 10) & 0x1F, m = b & 0x3FF;
  if (e == 31) return m ? std::nan("") : s * INFINITY;
  if (e == 0) return s * std::ldexp((double)m, -24);
  return s * std::ldexp(1.0 + m / 1024.0, e - 15);
}

uint16_t f16_round(double v) {
  const uint16_t sign = std::signbit(v) ? 0x8000 : 0;
  if (std::isnan(v)) return (uint16_t)(sign | 0x7E00);
  double a = std::fabs(v);
  if (a == 0.0) return sign;
  if (std::isinf(a)) return (uint16_t)(sign | 0x7C00);
  // 11 significant bits; normal exponents -14..15; below 2^-14 the spacing is 2^-24.
  int e = std::ilogb(a);
  int quantum_exp = (e < -14) ? -24 : e - 10;
  double r = std::ldexp(std::nearbyint(std::ldexp(a, -quantum_exp)), quantum_exp);  // ties to even
  if (r > 65504.0) return (uint16_t)(sign | 0x7C00);  // rounds past the largest finite half
  if (r == 0.0) return sign;
  if (r < 0x1p-14) return (uint16_t)(sign | (int)std::ldexp(r, 24));
  int E = std::ilogb(r);
  int mant = (int)((std::ldexp(r, -E) - 1.0) * 1024.0);
  return (uint16_t)(sign | ((E + 15) << 10) | mant);
}

// The activation element type: bf16 (the pages' type) or fp16.
struct Elem {
  double (*value)(uint16_t);
  uint16_t (*round)(double);
};
const Elem kBf16 = {bf16_value, bf16_round};
const Elem kF16 = {f16_value, f16_round};

uint8_t e4m3fn_round(double v) {
  if (std::isnan(v)) return 0x7F;
  const uint8_t sign = std::signbit(v) ? 0x80 : 0;
  double a = std::fabs(v);
  if (a > 448.0) a = 448.0;  // saturate (Inf included)
  if (a == 0.0) return sign;
  // 4 significant bits; normal exponents -6..8; below 2^-6 the spacing is 2^-9.
  int e = std::ilogb(a);
  int quantum_exp = (e < -6) ? -9 : e - 3;
  double r = std::ldexp(std::nearbyint(std::ldexp(a, -quantum_exp)), quantum_exp);
  if (r == 0.0) return sign;
  if (r < 0x1p-6) return (uint8_t)(sign | (int)std::ldexp(r, 9));  // subnormal: m * 2^-9
  int E = std::ilogb(r);
  int mant = (int)((std::ldexp(r, -E) - 1.0) * 8.0);
  return (uint8_t)(sign | ((E + 7) << 3) | mant);
}

double e4m3fn_value(uint8_t c) {
  const double s = (c & 0x80) ? -1.0 : 1.0;
  const int e = (c >> 3) & 0xF, m = c & 7;
  if (e == 15 && m == 7) return std::nan("");
  if (e == 0) return s * std::ldexp((double)m, -9);
  return s * std::ldexp(1.0 + m / 8.0, e - 7);
}

uint8_t e2m1_round(double v) {
  if (std::isnan(v)) return 0x7;
  const uint8_t sign = std::signbit(v) ? 0x8 : 0;
  double a = std::fabs(v);
  if (a > 6.0) a = 6.0;  // saturate
  if (a == 0.0) return sign;
  // 2 significant bits; normal exponents 0..2; below 1 the spacing is 0.5.
  int e = std::ilogb(a);
  int quantum_exp = (e < 0) ? -1 : e - 1;
  double r = std::ldexp(std::nearbyint(std::ldexp(a, -quantum_exp)), quantum_exp);
  if (r < 1.0) return (uint8_t)(sign | (int)(r * 2.0));  // 0 or 0.5
  int E = std::ilogb(r);
  int mant = (int)((std::ldexp(r, -E) - 1.0) * 2.0);
  return (uint8_t)(sign | ((E + 1) << 1) | mant);
}

double e2m1_value(uint8_t c) {
  const double s = (c & 0x8) ? -1.0 : 1.0;
  const int e = (c >> 1) & 3, m = c & 1;
  if (e == 0) return s * 0.5 * m;
  return s * std::ldexp(1.0 + m / 2.0, e - 1);
}

uint8_t e8m0_for_amax(double amax) {
  if (!std::isfinite(amax)) return 0xFF;
  if (amax == 0.0) return 0;
  // E2M1's largest exponent is 2 (6 = 1.5 * 2^2): the block's largest
  // magnitude lands in [4, 8) after scaling by 2^-(floor(log2 amax) - 2).
  int b = std::ilogb(amax) - 2 + 127;
  if (b < 0) b = 0;
  if (b > 254) b = 254;
  return (uint8_t)b;
}

// Largest |v| over a granule of values; NaN if any element is NaN.
double granule_amax(const Elem& e, const uint16_t* y, int64_t n) {
  double amax = 0.0;
  for (int64_t i = 0; i < n; ++i) {
    double a = std::fabs(e.value(y[i]));
    if (std::isnan(a)) return a;
    if (a > amax) amax = a;
  }
  return amax;
}

// Residual add and RMSNorm of one row: fills r (the residual_out row) and y
// (the normalized row), each rounded once to the element type.
void add_and_norm_row(const Elem& e, const uint16_t* x, const uint16_t* res, const uint16_t* w,
                      int64_t H, float eps, uint16_t* r, uint16_t* y) {
  for (int64_t i = 0; i < H; ++i) r[i] = e.round(e.value(x[i]) + e.value(res[i]));
  double ss = 0.0;
  for (int64_t i = 0; i < H; ++i) {
    double v = e.value(r[i]);
    ss += v * v;
  }
  double rstd = 1.0 / std::sqrt(ss / (double)H + (double)eps);
  for (int64_t i = 0; i < H; ++i) y[i] = e.round(e.value(r[i]) * rstd * e.value(w[i]));
}

// FP8 quantization of one granule of the normalized row.
void quant_fp8_granule(const Elem& e, const uint16_t* y, int64_t n, uint8_t* q, float* scale) {
  double amax = granule_amax(e, y, n);
  float s = (float)amax / 448.0f;  // amax is a bf16 or fp16 value: the cast is exact
  *scale = s;
  for (int64_t i = 0; i < n; ++i) {
    double v = e.value(y[i]);
    if (amax == 0.0) {
      q[i] = std::signbit(v) ? 0x80 : 0x00;
    } else {
      float quotient = (float)v / s;  // IEEE fp32 division
      q[i] = e4m3fn_round((double)quotient);
    }
  }
}

// MXFP4 quantization of one 32-element block; codes[i] is the 4-bit code of
// element i (packed by the caller).
void quant_mxfp4_block(const Elem& e, const uint16_t* y, uint8_t* codes, uint8_t* scale_byte) {
  double amax = granule_amax(e, y, 32);
  uint8_t b = e8m0_for_amax(amax);
  *scale_byte = b;
  for (int i = 0; i < 32; ++i) {
    if (b == 0xFF) {
      codes[i] = 0;  // non-finite block: codes unspecified, written as 0
    } else {
      codes[i] = e2m1_round(std::ldexp(e.value(y[i]), -((int)b - 127)));  // exact scaling
    }
  }
}

bool bad_row_args(const void* x, int64_t ldx, const void* residual, int64_t ldr,
                  const void* weight, int64_t M, int64_t H, float eps,
                  const void* residual_out, const void* q_out, const void* scale_out) {
  if (M < 0 || H <= 0) return true;
  if (!(eps >= 0.0f)) return true;
  if (ldx < H || ldr < H) return true;
  if (M > 0 && (!x || !residual || !weight || !residual_out || !q_out || !scale_out)) return true;
  return false;
}

// The fused step for FP8 with one scale per `group` elements (group == H:
// per token), on rows of element type e.
int fused_fp8(const Elem& e, const uint16_t* x, int64_t ldx, const uint16_t* residual, int64_t ldr,
              const uint16_t* weight, int64_t M, int64_t H, float eps, int64_t group,
              uint16_t* residual_out, uint8_t* q_out, float* scale_out, uint16_t* y_out) {
  if (bad_row_args(x, ldx, residual, ldr, weight, M, H, eps, residual_out, q_out, scale_out))
    return 1;
  if (group <= 0 || H % group != 0) return 1;
  const int64_t G = H / group;
  std::vector<uint16_t> r(H), y(H);
  for (int64_t m = 0; m < M; ++m) {
    add_and_norm_row(e, x + m * ldx, residual + m * ldr, weight, H, eps, r.data(), y.data());
    for (int64_t g = 0; g < G; ++g)
      quant_fp8_granule(e, y.data() + g * group, group, q_out + m * H + g * group,
                        scale_out + m * G + g);
    std::memcpy(residual_out + m * H, r.data(), H * sizeof(uint16_t));
    if (y_out) std::memcpy(y_out + m * H, y.data(), H * sizeof(uint16_t));
  }
  return 0;
}

// Packs the 4-bit codes of one 32-element block into 16 bytes.
void pack_block(const uint8_t* codes, uint8_t* out) {
  for (int j = 0; j < 16; ++j) out[j] = (uint8_t)(codes[2 * j] | (codes[2 * j + 1] << 4));
}

int fused_mxfp4(const Elem& e, const uint16_t* x, int64_t ldx, const uint16_t* residual, int64_t ldr,
                const uint16_t* weight, int64_t M, int64_t H, float eps,
                uint16_t* residual_out, uint8_t* q_out, uint8_t* scale_out, uint16_t* y_out) {
  if (bad_row_args(x, ldx, residual, ldr, weight, M, H, eps, residual_out, q_out, scale_out))
    return 1;
  if (H % 32 != 0) return 1;
  const int64_t B = H / 32;
  std::vector<uint16_t> r(H), y(H);
  uint8_t codes[32];
  for (int64_t m = 0; m < M; ++m) {
    add_and_norm_row(e, x + m * ldx, residual + m * ldr, weight, H, eps, r.data(), y.data());
    for (int64_t b = 0; b < B; ++b) {
      quant_mxfp4_block(e, y.data() + b * 32, codes, scale_out + m * B + b);
      pack_block(codes, q_out + m * (H / 2) + b * 16);
    }
    std::memcpy(residual_out + m * H, r.data(), H * sizeof(uint16_t));
    if (y_out) std::memcpy(y_out + m * H, y.data(), H * sizeof(uint16_t));
  }
  return 0;
}

int quantize_fp8_rows(const Elem& e, const uint16_t* y, int64_t M, int64_t H, int64_t group,
                      uint8_t* q_out, float* scale_out) {
  if (M < 0 || H <= 0 || group <= 0 || H % group != 0) return 1;
  if (M > 0 && (!y || !q_out || !scale_out)) return 1;
  const int64_t G = H / group;
  for (int64_t m = 0; m < M; ++m)
    for (int64_t g = 0; g < G; ++g)
      quant_fp8_granule(e, y + m * H + g * group, group, q_out + m * H + g * group, scale_out + m * G + g);
  return 0;
}

int quantize_mxfp4_rows(const Elem& e, const uint16_t* y, int64_t M, int64_t H, uint8_t* q_out,
                        uint8_t* scale_out) {
  if (M < 0 || H <= 0 || H % 32 != 0) return 1;
  if (M > 0 && (!y || !q_out || !scale_out)) return 1;
  const int64_t B = H / 32;
  uint8_t codes[32];
  for (int64_t m = 0; m < M; ++m)
    for (int64_t b = 0; b < B; ++b) {
      quant_mxfp4_block(e, y + m * H + b * 32, codes, scale_out + m * B + b);
      pack_block(codes, q_out + m * (H / 2) + b * 16);
    }
  return 0;
}

// The same steps with the scales written column-major: scale (m, g) at
// scale_out[g * ld_scale + m], ld_scale >= M.  A layout only: the values are
// those of the row-major functions above, stored transposed.
template <typename S>
bool bad_transposed_scales(const S* scale_out, int64_t M, int64_t ld_scale) {
  return M < 0 || ld_scale < M || ld_scale < 1 || (M > 0 && !scale_out);
}

template <typename S>
void store_transposed(const std::vector<S>& row_major, int64_t M, int64_t G, S* scale_out, int64_t ld_scale) {
  for (int64_t m = 0; m < M; ++m)
    for (int64_t g = 0; g < G; ++g) scale_out[g * ld_scale + m] = row_major[m * G + g];
}

int fused_fp8_tscale(const Elem& e, const uint16_t* x, int64_t ldx, const uint16_t* residual, int64_t ldr,
                     const uint16_t* weight, int64_t M, int64_t H, float eps, int64_t group,
                     uint16_t* residual_out, uint8_t* q_out, float* scale_out, int64_t ld_scale,
                     uint16_t* y_out) {
  if (bad_transposed_scales(scale_out, M, ld_scale) || group <= 0 || H <= 0 || H % group != 0) return 1;
  const int64_t G = H / group;
  std::vector<float> rm((size_t)(M > 0 ? M : 0) * G + 1);
  int rc = fused_fp8(e, x, ldx, residual, ldr, weight, M, H, eps, group, residual_out, q_out, rm.data(), y_out);
  if (rc != 0) return rc;
  store_transposed(rm, M, G, scale_out, ld_scale);
  return 0;
}

int fused_mxfp4_tscale(const Elem& e, const uint16_t* x, int64_t ldx, const uint16_t* residual, int64_t ldr,
                       const uint16_t* weight, int64_t M, int64_t H, float eps, uint16_t* residual_out,
                       uint8_t* q_out, uint8_t* scale_out, int64_t ld_scale, uint16_t* y_out) {
  if (bad_transposed_scales(scale_out, M, ld_scale) || H <= 0 || H % 32 != 0) return 1;
  const int64_t B = H / 32;
  std::vector<uint8_t> rm((size_t)(M > 0 ? M : 0) * B + 1);
  int rc = fused_mxfp4(e, x, ldx, residual, ldr, weight, M, H, eps, residual_out, q_out, rm.data(), y_out);
  if (rc != 0) return rc;
  store_transposed(rm, M, B, scale_out, ld_scale);
  return 0;
}

}  // namespace

extern "C" {

double rq_ref_f64_from_bf16(uint16_t b) { return bf16_value(b); }
uint16_t rq_ref_bf16_from_f64(double v) { return bf16_round(v); }
uint8_t rq_ref_e4m3fn_from_f64(double v) { return e4m3fn_round(v); }
double rq_ref_f64_from_e4m3fn(uint8_t c) { return e4m3fn_value(c); }
uint8_t rq_ref_e2m1_from_f64(double v) { return e2m1_round(v); }
double rq_ref_f64_from_e2m1(uint8_t c) { return e2m1_value(c); }
uint8_t rq_ref_e8m0_from_amax(double amax) { return e8m0_for_amax(amax); }
double rq_ref_f64_from_e8m0(uint8_t b) {
  return b == 0xFF ? std::nan("") : std::ldexp(1.0, (int)b - 127);
}


double rq_ref_f64_from_f16(uint16_t b) { return f16_value(b); }
uint16_t rq_ref_f16_from_f64(double v) { return f16_round(v); }

#define RQ_REF_ROW_EXPORTS(SUFFIX, ELEM)                                                            \
  int rq_ref_rmsnorm_quant_fp8_per_token##SUFFIX(                                                   \
      const uint16_t* x, int64_t ldx, const uint16_t* residual, int64_t ldr, const uint16_t* weight, \
      int64_t M, int64_t H, float eps, uint16_t* residual_out, uint8_t* q_out, float* scale_out,    \
      uint16_t* y_out) {                                                                           \
    return fused_fp8(ELEM, x, ldx, residual, ldr, weight, M, H, eps, H, residual_out, q_out,        \
                     scale_out, y_out);                                                            \
  }                                                                                                \
  int rq_ref_rmsnorm_quant_fp8_per_group##SUFFIX(                                                   \
      const uint16_t* x, int64_t ldx, const uint16_t* residual, int64_t ldr, const uint16_t* weight, \
      int64_t M, int64_t H, float eps, int64_t group, uint16_t* residual_out, uint8_t* q_out,       \
      float* scale_out, uint16_t* y_out) {                                                         \
    return fused_fp8(ELEM, x, ldx, residual, ldr, weight, M, H, eps, group, residual_out, q_out,    \
                     scale_out, y_out);                                                            \
  }                                                                                                \
  int rq_ref_rmsnorm_quant_mxfp4##SUFFIX(                                                           \
      const uint16_t* x, int64_t ldx, const uint16_t* residual, int64_t ldr, const uint16_t* weight, \
      int64_t M, int64_t H, float eps, uint16_t* residual_out, uint8_t* q_out, uint8_t* scale_out,  \
      uint16_t* y_out) {                                                                           \
    return fused_mxfp4(ELEM, x, ldx, residual, ldr, weight, M, H, eps, residual_out, q_out,         \
                       scale_out, y_out);                                                          \
  }                                                                                                \
  int rq_ref_quantize_fp8##SUFFIX(const uint16_t* y, int64_t M, int64_t H, int64_t group,           \
                                  uint8_t* q_out, float* scale_out) {                              \
    return quantize_fp8_rows(ELEM, y, M, H, group, q_out, scale_out);                              \
  }                                                                                                \
  int rq_ref_quantize_mxfp4##SUFFIX(const uint16_t* y, int64_t M, int64_t H, uint8_t* q_out,        \
                                    uint8_t* scale_out) {                                          \
    return quantize_mxfp4_rows(ELEM, y, M, H, q_out, scale_out);                                   \
  }                                                                                                \
  int rq_ref_rmsnorm_quant_fp8_per_group_tscale##SUFFIX(                                            \
      const uint16_t* x, int64_t ldx, const uint16_t* residual, int64_t ldr, const uint16_t* weight, \
      int64_t M, int64_t H, float eps, int64_t group, uint16_t* residual_out, uint8_t* q_out,       \
      float* scale_out, int64_t ld_scale, uint16_t* y_out) {                                       \
    return fused_fp8_tscale(ELEM, x, ldx, residual, ldr, weight, M, H, eps, group, residual_out,    \
                            q_out, scale_out, ld_scale, y_out);                                    \
  }                                                                                                \
  int rq_ref_rmsnorm_quant_mxfp4_tscale##SUFFIX(                                                    \
      const uint16_t* x, int64_t ldx, const uint16_t* residual, int64_t ldr, const uint16_t* weight, \
      int64_t M, int64_t H, float eps, uint16_t* residual_out, uint8_t* q_out, uint8_t* scale_out,  \
      int64_t ld_scale, uint16_t* y_out) {                                                         \
    return fused_mxfp4_tscale(ELEM, x, ldx, residual, ldr, weight, M, H, eps, residual_out, q_out,  \
                              scale_out, ld_scale, y_out);                                         \
  }

RQ_REF_ROW_EXPORTS(, kBf16)
RQ_REF_ROW_EXPORTS(_f16, kF16)

int rq_ref_qk_gemma_rmsnorm_gate(
    const uint16_t* qg, int64_t ld_qg, const uint16_t* k, int64_t ld_k,
    const uint16_t* q_w, const uint16_t* k_w, int64_t T, int64_t Hq, int64_t Hk,
    int64_t D, float eps, uint16_t* q_out, uint16_t* k_out, uint16_t* gate_out) {
  if (T < 0 || Hq < 0 || Hk < 0 || D <= 0 || !(eps >= 0.0f)) return 1;
  if (ld_qg < 2 * Hq * D || ld_k < Hk * D) return 1;
  if (T > 0 && (!qg || !k || !q_w || !k_w || !q_out || !k_out || !gate_out)) return 1;
  // GemmaRMSNorm of one head's D values: v * rstd * (1 + w), rounded once.
  auto gemma_norm = [D, eps](const uint16_t* v, const uint16_t* w, uint16_t* out) {
    double ss = 0.0;
    for (int64_t i = 0; i < D; ++i) ss += bf16_value(v[i]) * bf16_value(v[i]);
    double rstd = 1.0 / std::sqrt(ss / (double)D + (double)eps);
    for (int64_t i = 0; i < D; ++i)
      out[i] = bf16_round(bf16_value(v[i]) * rstd * (1.0 + bf16_value(w[i])));
  };
  for (int64_t t = 0; t < T; ++t) {
    for (int64_t h = 0; h < Hq; ++h) {
      const uint16_t* q_part = qg + t * ld_qg + 2 * D * h;
      const uint16_t* gate_part = q_part + D;
      gemma_norm(q_part, q_w, q_out + (t * Hq + h) * D);
      std::memcpy(gate_out + (t * Hq + h) * D, gate_part, D * sizeof(uint16_t));
    }
    for (int64_t h = 0; h < Hk; ++h)
      gemma_norm(k + t * ld_k + D * h, k_w, k_out + (t * Hk + h) * D);
  }
  return 0;
}

// The QK step followed by FP8 quantization of the normalized q and k, one
// scale per head of each token: the bf16 heads of the step above, each
// quantized as one granule of D values by the per-token FP8 rule (scale =
// amax / 448).  The pages fuse a downstream quantization of the attention
// inputs without giving its granule; one head of one token is the plainest
// granule of that data.
int rq_ref_qk_gemma_rmsnorm_gate_fp8(
    const uint16_t* qg, int64_t ld_qg, const uint16_t* k, int64_t ld_k,
    const uint16_t* q_w, const uint16_t* k_w, int64_t T, int64_t Hq, int64_t Hk,
    int64_t D, float eps, uint8_t* q_codes, float* q_scale, uint8_t* k_codes, float* k_scale,
    uint16_t* gate_out) {
  if (T > 0 && (!q_codes || !q_scale || !k_codes || !k_scale)) return 1;
  // At least one element each, so that a side with no heads still passes a
  // non-null buffer to the step above.
  const size_t nq = (size_t)(T > 0 ? T : 0) * (size_t)(Hq > 0 ? Hq : 0) * (size_t)D;
  const size_t nk = (size_t)(T > 0 ? T : 0) * (size_t)(Hk > 0 ? Hk : 0) * (size_t)D;
  std::vector<uint16_t> q_bf16(nq > 0 ? nq : 1), k_bf16(nk > 0 ? nk : 1);
  int rc = rq_ref_qk_gemma_rmsnorm_gate(qg, ld_qg, k, ld_k, q_w, k_w, T, Hq, Hk, D, eps, q_bf16.data(),
                                        k_bf16.data(), gate_out);
  if (rc != 0) return rc;
  rc = quantize_fp8_rows(kBf16, q_bf16.data(), T * Hq, D, D, q_codes, q_scale);
  if (rc != 0) return rc;
  return quantize_fp8_rows(kBf16, k_bf16.data(), T * Hk, D, D, k_codes, k_scale);
}

// The QK step followed by MXFP4 quantization of the normalized q and k: each
// bf16 head is a row of D values quantized with one E8M0 scale per 32
// elements, exactly as the rows of the fused step (D a multiple of 32).
int rq_ref_qk_gemma_rmsnorm_gate_mxfp4(
    const uint16_t* qg, int64_t ld_qg, const uint16_t* k, int64_t ld_k,
    const uint16_t* q_w, const uint16_t* k_w, int64_t T, int64_t Hq, int64_t Hk,
    int64_t D, float eps, uint8_t* q_codes, uint8_t* q_scale, uint8_t* k_codes, uint8_t* k_scale,
    uint16_t* gate_out) {
  if (D <= 0 || D % 32 != 0) return 1;
  if (T > 0 && (!q_codes || !q_scale || !k_codes || !k_scale)) return 1;
  const size_t nq = (size_t)(T > 0 ? T : 0) * (size_t)(Hq > 0 ? Hq : 0) * (size_t)D;
  const size_t nk = (size_t)(T > 0 ? T : 0) * (size_t)(Hk > 0 ? Hk : 0) * (size_t)D;
  std::vector<uint16_t> q_bf16(nq > 0 ? nq : 1), k_bf16(nk > 0 ? nk : 1);
  int rc = rq_ref_qk_gemma_rmsnorm_gate(qg, ld_qg, k, ld_k, q_w, k_w, T, Hq, Hk, D, eps, q_bf16.data(),
                                        k_bf16.data(), gate_out);
  if (rc != 0) return rc;
  rc = quantize_mxfp4_rows(kBf16, q_bf16.data(), T * Hq, D, q_codes, q_scale);
  if (rc != 0) return rc;
  return quantize_mxfp4_rows(kBf16, k_bf16.data(), T * Hk, D, k_codes, k_scale);
}

}  // extern "C"
