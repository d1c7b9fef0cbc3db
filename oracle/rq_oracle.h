/*
 * rq_oracle.h -- plain CPU oracle for the fused residual-add -> RMSNorm ->
 * activation-quantization step and the QK GemmaRMSNorm + gate de-interleave.
 *
 * TEST INFRASTRUCTURE ONLY.  This header and librq_oracle.so are the checker
 * the HIP library is compared against.  Only the test suite, the smoke check
 * and the benchmark's CPU-baseline leg may load it.  It shares no code, header,
 * constant or table with the HIP library, and includes nothing from it.
 *
 * Everything is host memory, row-major, one row per token.  bf16 values are
 * passed as their raw 16-bit patterns (uint16_t).
 *
 * Sources (web pages; cited by page and section):
 *  - sglang PR #29723, "fused AllReduce + RMSNorm + quant (per-token FP8,
 *    MXFP4) on AMD": Motivation, Key changes, Accuracy Tests.  The fused step
 *    must equal the unfused sequence residual-add -> RMSNorm -> quantize with
 *    bf16 tensors between the steps, and returns (codes, residual_out,
 *    per-token scale of shape (M, 1)), optionally with a bf16 side output
 *    (review comments on emit_bf16, "Applicability").
 *  - sgl-amd-mono PR #26 "[Feat] [MI355X] muse_spark: Whole-layer monokernels
 *    for Muse Spark", commit notes: MXFP4 blocks are a pure function of the
 *    bf16 normalized row.
 *  - sglang PR #27656 "[AMD][Perf] Fuse QK RMSNorm + gate extraction Triton
 *    kernel for Qwen3.5 on HIP": Motivation, Modifications (interleaved
 *    [q_h0, gate_h0, q_h1, gate_h1, ...] input, GemmaRMSNorm on q and k,
 *    contiguous q, k, gate outputs; k may be a strided view per the review).
 * The pages do not print the quantization formulas; the workload statement
 * fixes scale = amax / 448 (FP8) and E8M0 exponent floor(log2 amax) - 2
 * (MXFP4, one scale per 32 elements).
 *
 * Pins: every function here is checked by the CPU tests against closed forms,
 * format tables, exhaustive searches, hand-derived goldens and an independent
 * numpy formulation (with planted mistakes as negative controls).  Parity
 * unpinned against the pages themselves, which print no outputs: the rounding
 * order inside RMSNorm (one rounding of r * rstd * w, fp64 here), the FP8
 * flavour (OCP E4M3FN, read from the /448), the E8M0 rule without a mantissa
 * round-up, the scale layouts, and the granule of the quantized QK variants
 * (one FP8 scale per head of a token; MXFP4 heads as rows of D values).
 *
 * Return value of the row functions: 0 on success, 1 on an invalid argument
 * (null pointer with M > 0, negative size, leading dimension below the row
 * length, H not divisible by the granule).  Nothing is written on failure.
 */
#ifndef RQ_ORACLE_H
#define RQ_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- number formats (exported so the tests can pin them one by one) ---- */

/* bf16 bits -> exact value. */
double rq_ref_f64_from_bf16(uint16_t b);
/* Round a double to the nearest bf16 (ties to even), overflow -> +-Inf, NaN -> 0x7FC0|sign. */
uint16_t rq_ref_bf16_from_f64(double v);

/* IEEE binary16 (fp16) bits -> exact value, and rounding of a double to the
 * nearest fp16 (ties to even, |v| rounding past 65504 -> +-Inf). */
double rq_ref_f64_from_f16(uint16_t b);
uint16_t rq_ref_f16_from_f64(double v);

/* OCP FP8 E4M3FN: bias 7, no infinities, 0x7F/0xFF NaN, max 448.
 * Nearest, ties to even; |v| > 448 saturates to +-448; NaN -> 0x7F. */
uint8_t rq_ref_e4m3fn_from_f64(double v);
double rq_ref_f64_from_e4m3fn(uint8_t c);

/* FP4 E2M1 (4-bit code, sign in bit 3): values 0, .5, 1, 1.5, 2, 3, 4, 6.
 * Nearest, ties to even; |v| > 6 saturates to +-6.  NaN -> 0x7 (unspecified). */
uint8_t rq_ref_e2m1_from_f64(double v);
double rq_ref_f64_from_e2m1(uint8_t c);

/* E8M0 shared exponent for a block whose largest magnitude is amax:
 * floor(log2 amax) - 2 + 127 clamped to [0, 254]; amax == 0 -> 0;
 * non-finite amax -> 255 (the E8M0 NaN). */
uint8_t rq_ref_e8m0_from_amax(double amax);
double rq_ref_f64_from_e8m0(uint8_t b);

/* ---- the fused step ---- */

/* residual_out = bf16(x + residual); y = bf16(residual_out * rstd * weight);
 * per-token FP8: scale[m] = fp32(amax_m) / 448 (IEEE fp32 division),
 * q = e4m3fn(y / scale).  y_out may be NULL. */
int rq_ref_rmsnorm_quant_fp8_per_token(
    const uint16_t* x, int64_t ldx, const uint16_t* residual, int64_t ldr,
    const uint16_t* weight, int64_t M, int64_t H, float eps,
    uint16_t* residual_out, uint8_t* q_out, float* scale_out, uint16_t* y_out);

/* Same, one scale per `group` consecutive elements of a row;
 * scale_out is row-major [M, H / group]. */
int rq_ref_rmsnorm_quant_fp8_per_group(
    const uint16_t* x, int64_t ldx, const uint16_t* residual, int64_t ldr,
    const uint16_t* weight, int64_t M, int64_t H, float eps, int64_t group,
    uint16_t* residual_out, uint8_t* q_out, float* scale_out, uint16_t* y_out);

/* MXFP4: one E8M0 byte per 32 elements (scale_out row-major [M, H / 32]),
 * E2M1 codes of y * 2^-(byte - 127), two per byte, element 2j in the low
 * nibble of byte j (q_out row-major [M, H / 2]). */
int rq_ref_rmsnorm_quant_mxfp4(
    const uint16_t* x, int64_t ldx, const uint16_t* residual, int64_t ldr,
    const uint16_t* weight, int64_t M, int64_t H, float eps,
    uint16_t* residual_out, uint8_t* q_out, uint8_t* scale_out, uint16_t* y_out);

/* ---- the quantize step alone (the last launch of the unfused sequence) ---- */

/* FP8 quantization of a bf16 tensor y [M, H]: one scale per `group`
 * consecutive elements (group == H: per token), same rules as above. */
int rq_ref_quantize_fp8(const uint16_t* y, int64_t M, int64_t H, int64_t group,
                        uint8_t* q_out, float* scale_out);
/* MXFP4 quantization of a bf16 tensor y [M, H], same rules as above. */
int rq_ref_quantize_mxfp4(const uint16_t* y, int64_t M, int64_t H,
                          uint8_t* q_out, uint8_t* scale_out);

/* ---- fp16 rows ----
 * The same functions on IEEE fp16 activations (x, residual, weight,
 * residual_out and y are fp16; every rounding is to fp16 instead of bf16),
 * the activation dtype carried through the step as the review of sglang
 * PR #29723 asks.  Same arguments and results otherwise. */
int rq_ref_rmsnorm_quant_fp8_per_token_f16(
    const uint16_t* x, int64_t ldx, const uint16_t* residual, int64_t ldr,
    const uint16_t* weight, int64_t M, int64_t H, float eps,
    uint16_t* residual_out, uint8_t* q_out, float* scale_out, uint16_t* y_out);
int rq_ref_rmsnorm_quant_fp8_per_group_f16(
    const uint16_t* x, int64_t ldx, const uint16_t* residual, int64_t ldr,
    const uint16_t* weight, int64_t M, int64_t H, float eps, int64_t group,
    uint16_t* residual_out, uint8_t* q_out, float* scale_out, uint16_t* y_out);
int rq_ref_rmsnorm_quant_mxfp4_f16(
    const uint16_t* x, int64_t ldx, const uint16_t* residual, int64_t ldr,
    const uint16_t* weight, int64_t M, int64_t H, float eps,
    uint16_t* residual_out, uint8_t* q_out, uint8_t* scale_out, uint16_t* y_out);
int rq_ref_quantize_fp8_f16(const uint16_t* y, int64_t M, int64_t H, int64_t group,
                            uint8_t* q_out, float* scale_out);
int rq_ref_quantize_mxfp4_f16(const uint16_t* y, int64_t M, int64_t H,
                              uint8_t* q_out, uint8_t* scale_out);

/* ---- transposed scales ----
 * The fused per-group FP8 and MXFP4 steps with the scales stored
 * column-major for consumers that read them per group (the scale transpose
 * for the preshuffled-weight GEMM named in the review of sglang PR #29723):
 * scale (m, g) at scale_out[g * ld_scale + m], ld_scale >= M; scale_out holds
 * (H / granule - 1) * ld_scale + M values.  Everything else as above; the
 * _f16 names take fp16 rows. */
int rq_ref_rmsnorm_quant_fp8_per_group_tscale(
    const uint16_t* x, int64_t ldx, const uint16_t* residual, int64_t ldr,
    const uint16_t* weight, int64_t M, int64_t H, float eps, int64_t group,
    uint16_t* residual_out, uint8_t* q_out, float* scale_out, int64_t ld_scale, uint16_t* y_out);
int rq_ref_rmsnorm_quant_mxfp4_tscale(
    const uint16_t* x, int64_t ldx, const uint16_t* residual, int64_t ldr,
    const uint16_t* weight, int64_t M, int64_t H, float eps,
    uint16_t* residual_out, uint8_t* q_out, uint8_t* scale_out, int64_t ld_scale, uint16_t* y_out);
int rq_ref_rmsnorm_quant_fp8_per_group_tscale_f16(
    const uint16_t* x, int64_t ldx, const uint16_t* residual, int64_t ldr,
    const uint16_t* weight, int64_t M, int64_t H, float eps, int64_t group,
    uint16_t* residual_out, uint8_t* q_out, float* scale_out, int64_t ld_scale, uint16_t* y_out);
int rq_ref_rmsnorm_quant_mxfp4_tscale_f16(
    const uint16_t* x, int64_t ldx, const uint16_t* residual, int64_t ldr,
    const uint16_t* weight, int64_t M, int64_t H, float eps,
    uint16_t* residual_out, uint8_t* q_out, uint8_t* scale_out, int64_t ld_scale, uint16_t* y_out);

/* ---- the QK variant ---- */

/* qg: [T, ld_qg] with per-token layout [q_0 | gate_0 | q_1 | gate_1 | ...],
 * each part D wide (ld_qg >= 2 * Hq * D).  k: [T, ld_k] with Hk heads of D
 * (ld_k >= Hk * D).  GemmaRMSNorm over each head's D values with weight
 * (1 + w).  Outputs contiguous: q_out [T, Hq, D], k_out [T, Hk, D],
 * gate_out [T, Hq, D] (gate copied bit for bit). */
int rq_ref_qk_gemma_rmsnorm_gate(
    const uint16_t* qg, int64_t ld_qg, const uint16_t* k, int64_t ld_k,
    const uint16_t* q_w, const uint16_t* k_w, int64_t T, int64_t Hq, int64_t Hk,
    int64_t D, float eps, uint16_t* q_out, uint16_t* k_out, uint16_t* gate_out);

/* The QK step, then FP8 quantization of each normalized head: the bf16 q and
 * k heads of rq_ref_qk_gemma_rmsnorm_gate, each one granule of D values with
 * the per-token rule (scale = fp32(amax) / 448, q = e4m3fn(v / scale)).
 * q_codes [T, Hq, D] and k_codes [T, Hk, D] E4M3FN bytes; q_scale [T, Hq] and
 * k_scale [T, Hk] fp32; gate_out as above. */
int rq_ref_qk_gemma_rmsnorm_gate_fp8(
    const uint16_t* qg, int64_t ld_qg, const uint16_t* k, int64_t ld_k,
    const uint16_t* q_w, const uint16_t* k_w, int64_t T, int64_t Hq, int64_t Hk,
    int64_t D, float eps, uint8_t* q_codes, float* q_scale, uint8_t* k_codes, float* k_scale,
    uint16_t* gate_out);

/* The QK step, then MXFP4 quantization of each normalized head: each bf16
 * head is a row of D values (D a multiple of 32) quantized with one E8M0
 * byte per 32 elements, as in rq_ref_rmsnorm_quant_mxfp4.
 * q_codes [T, Hq, D / 2] and k_codes [T, Hk, D / 2] packed E2M1 (element 2j
 * in the low nibble of byte j); q_scale [T, Hq, D / 32] and
 * k_scale [T, Hk, D / 32] E8M0 bytes; gate_out as above. */
int rq_ref_qk_gemma_rmsnorm_gate_mxfp4(
    const uint16_t* qg, int64_t ld_qg, const uint16_t* k, int64_t ld_k,
    const uint16_t* q_w, const uint16_t* k_w, int64_t T, int64_t Hq, int64_t Hk,
    int64_t D, float eps, uint8_t* q_codes, uint8_t* q_scale, uint8_t* k_codes, uint8_t* k_scale,
    uint16_t* gate_out);

#ifdef __cplusplus
}
#endif

#endif /* RQ_ORACLE_H */
