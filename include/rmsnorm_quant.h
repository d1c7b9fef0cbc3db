/*
 * rmsnorm_quant.h -- C ABI of librmsnorm_quant.so, the MI355X (gfx950) library
 * for the fused residual-add -> RMSNorm -> activation-quantization step and the
 * QK GemmaRMSNorm + gate de-interleave step of LLM decoder layers.
 *
 * What is computed (per row = per token, row-major tensors):
 *
 *   residual_out = bf16(x + residual)                      (one rounding)
 *   rstd         = 1 / sqrt(mean(residual_out^2) + eps)    (mean over H)
 *   y            = bf16(residual_out * rstd * weight)      (one rounding)
 *   then y is quantized in one of three formats.
 *
 * sglang PR #29723 (fused AllReduce + RMSNorm + per-token FP8 / MXFP4 quant on
 * AMD), Motivation: the unfused sequence is residual add -> RMSNorm ->
 * quantize in separate launches with bf16 tensors between them; Accuracy
 * Tests: the fused kernel is numerically equivalent to that sequence; Key
 * changes: the call returns (codes, residual_out, per-token scale of shape
 * (M, 1)) or tells the caller it cannot fuse.  The all-reduce the page fuses in
 * front of the residual add is not part of this library (one GPU); x is the
 * already-reduced activation.
 *
 * Conventions shared by every entry point:
 *  - bf16 tensors are passed as uint16_t bit patterns.  The calls with an
 *    _f16 suffix take and return IEEE fp16 instead; no call promotes one type
 *    to the other.
 *  - All tensor pointers are DEVICE pointers owned by the caller.  The library
 *    allocates nothing, never synchronizes the host and keeps no state besides
 *    a per-device cache of the architecture check.  Every call only enqueues
 *    kernels on `stream` (a hipStream_t; NULL = the null stream), so calls may
 *    be captured into a hipGraph.  The architecture check reads the current
 *    HIP device: the stream and every pointer must belong to that device
 *    (the library cannot see where a pointer or a stream lives).
 *  - Inputs x and residual may be strided views (row stride ldx / ldr in
 *    elements); every output is contiguous, except the column-major scale
 *    arrays of the _tscale calls, which take a leading dimension.
 *    residual_out may alias residual
 *    exactly (in place) when ldr == H; any other overlap between an output and
 *    any other buffer is rejected.
 *  - Errors are decided by deterministic checks before anything is enqueued,
 *    so on any error return nothing has been written:
 *      RQ_ERR_INVALID      a null pointer with M > 0, a negative size,
 *                          ld < row length, eps negative or NaN, overlapping
 *                          buffers, a stride or size whose extent could not
 *                          be a real buffer (2^48 bytes or more);
 *      RQ_ERR_UNSUPPORTED  a row start is not 16-byte aligned, H % 8 != 0,
 *                          H above RQ_MAX_HIDDEN, a granule that does not
 *                          divide H, an unsupported group size, or M (or T)
 *                          above 2^31 - 1.  This is the "cannot fuse, use
 *                          the unfused path" answer of PR #29723.
 *      RQ_ERR_DEVICE       the current HIP device is not an MI355X (gfx950).
 *                          Every entry point, fused or unfused, returns it
 *                          there, so it is an error, not a fallback signal.
 *      RQ_ERR_HIP          the kernel launch itself failed, or the HIP
 *                          runtime could not name the current device.
 *    Faults inside a kernel surface at the caller's next synchronization.
 *  - M == 0 (or T == 0) returns RQ_OK and launches nothing.
 *  - A call is one launch per step unless its grid would exceed 2^31
 *    work-items (for instance more than 2^25 rows at H <= 1024, or 2^21 rows
 *    at H = 16384); then the rows (or heads) are split over several launches
 *    of the same kernel, with the same results.  RQ_ERR_HIP from a later
 *    launch leaves the earlier ones enqueued.
 */
#ifndef RMSNORM_QUANT_H
#define RMSNORM_QUANT_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* C++ includers see a fixed underlying type (int), so that any status value a
 * C caller can hold (rq_status_string takes unknown codes too) is a valid
 * value of the enumeration in C++ as well; the size and calling convention are
 * those of the C enum. */
#ifdef __cplusplus
typedef enum rq_status : int {
#else
typedef enum rq_status {
#endif
  RQ_OK = 0,
  RQ_ERR_INVALID = 1,
  RQ_ERR_UNSUPPORTED = 2,
  RQ_ERR_HIP = 3,
  RQ_ERR_DEVICE = 4
} rq_status;

/* Largest row length the fused row kernels accept (the row is held in
 * registers).  Larger H returns RQ_ERR_UNSUPPORTED. */
#define RQ_MAX_HIDDEN 16384
/* Largest head dimension of qk_gemma_rmsnorm_gate. */
#define RQ_MAX_HEAD_DIM 512

/* Fused residual add + RMSNorm + per-token FP8 quantization.
 * sglang PR #29723, Key changes: tensor_model_parallel_fused_allreduce_
 * rmsnorm_quant_per_token returns (fp8_output, residual_out,
 * per_token_scale (M, 1)); review notes and "Applicability": an optional bf16
 * side output for consumers that cannot take the quantized tuple.
 *
 *  x          [M, ldx] bf16, first H columns used (the reduced activation)
 *  residual   [M, ldr] bf16
 *  weight     [H] bf16 (RMSNorm gamma)
 *  eps        added to the mean of squares inside the square root
 *  residual_out [M, H] bf16 out: bf16(x + residual)
 *  q_out      [M, H] uint8 out: OCP FP8 E4M3FN codes of y / scale
 *             (nearest-even; y / scale is an IEEE fp32 quotient)
 *  scale_out  [M] fp32 out: scale = fp32(max |y| over the row) / 448;
 *             an all-zero row has scale 0 and codes 0x00 / 0x80 (sign of zero)
 *             when eps > 0; with eps = 0 its y is 0 * (1/0), NaN, and so are
 *             its scale and codes
 *  y_out      [M, H] bf16 out or NULL: the normalized row y
 *  stream     hipStream_t
 */
rq_status rmsnorm_quant_fp8_per_token(
    const uint16_t* x, int64_t ldx, const uint16_t* residual, int64_t ldr,
    const uint16_t* weight, int64_t M, int64_t H, float eps,
    uint16_t* residual_out, uint8_t* q_out, float* scale_out, uint16_t* y_out,
    void* stream);

/* Fused residual add + RMSNorm + per-group FP8 quantization (the pre-existing
 * per-group variant of sglang PR #29723, Motivation).  As the per-token call,
 * but one scale per `group` consecutive elements of a row, groups starting at
 * column 0:
 *  group      one of 32, 64, 128, 256, 512; must divide H
 *  scale_out  [M, H / group] fp32 row-major
 */
rq_status rmsnorm_quant_fp8_per_group(
    const uint16_t* x, int64_t ldx, const uint16_t* residual, int64_t ldr,
    const uint16_t* weight, int64_t M, int64_t H, float eps, int64_t group,
    uint16_t* residual_out, uint8_t* q_out, float* scale_out, uint16_t* y_out,
    void* stream);

/* Fused residual add + RMSNorm + MXFP4 quantization (sglang PR #29723: the
 * MXFP4 variant with a direct MXFP4 epilogue; sgl-amd-mono PR #26 commit notes:
 * the MXFP4 blocks are a pure function of the bf16 normalized row).
 *  H          must be a multiple of 32
 *  q_out      [M, H / 2] uint8 out: FP4 E2M1 codes, two per byte, element 2j
 *             in the low nibble of byte j; code = E2M1(y * 2^-(s - 127)),
 *             nearest-even, saturating at 6
 *  scale_out  [M, H / 32] uint8 out: E8M0 byte s per 32-element block,
 *             s = clamp(floor(log2 max|y|) - 2 + 127, 0, 254); an all-zero
 *             block has s = 0 and codes 0x0 / 0x8 (sign of zero); a block
 *             holding NaN or Inf has s = 255 and unspecified codes
 */
rq_status rmsnorm_quant_mxfp4(
    const uint16_t* x, int64_t ldx, const uint16_t* residual, int64_t ldr,
    const uint16_t* weight, int64_t M, int64_t H, float eps,
    uint16_t* residual_out, uint8_t* q_out, uint8_t* scale_out, uint16_t* y_out,
    void* stream);

/* ---- The unfused sequence, one launch per step ----
 * sglang PR #29723, Motivation: without fusion the step runs as separate
 * launches with bf16 tensors between them (the all-reduce, RMSNorm with the
 * residual add, then the quantization); Speed Tests: the fused kernel is
 * benchmarked against that sequence; "Applicability": a consumer that cannot
 * take the quantized tuple needs the bf16 row.  These entry points are those
 * launches on one GPU.  Their results equal the fused entry points' bit for
 * bit: rmsnorm_residual_bf16 followed by quantize_* gives exactly the codes
 * and scales of rmsnorm_quant_* (the same kernel code computes y).
 */

/* residual_out = bf16(x + residual); y_out = bf16(residual_out * rstd * weight).
 * Arguments, layout, aliasing and errors as rmsnorm_quant_fp8_per_token;
 * y_out [M, H] bf16 is required. */
rq_status rmsnorm_residual_bf16(
    const uint16_t* x, int64_t ldx, const uint16_t* residual, int64_t ldr,
    const uint16_t* weight, int64_t M, int64_t H, float eps,
    uint16_t* residual_out, uint16_t* y_out, void* stream);

/* Quantize a bf16 tensor y [M, ldy] (first H columns) with the rules and
 * output layouts of rmsnorm_quant_fp8_per_token / _fp8_per_group / _mxfp4.
 * Outputs must not overlap y. */
rq_status quantize_fp8_per_token(
    const uint16_t* y, int64_t ldy, int64_t M, int64_t H,
    uint8_t* q_out, float* scale_out, void* stream);
rq_status quantize_fp8_per_group(
    const uint16_t* y, int64_t ldy, int64_t M, int64_t H, int64_t group,
    uint8_t* q_out, float* scale_out, void* stream);
rq_status quantize_mxfp4(
    const uint16_t* y, int64_t ldy, int64_t M, int64_t H,
    uint8_t* q_out, uint8_t* scale_out, void* stream);

/* ---- fp16 activations ----
 * The review of sglang PR #29723 asks that the activation dtype be carried
 * through the fused tuple rather than silently promoted to bf16.  These take
 * IEEE fp16 x, residual and weight (as uint16_t bits) and return fp16
 * residual_out and y, with every rounding to fp16 instead of bf16; codes,
 * scales, layouts, aliasing and errors are exactly those of the bf16 calls of
 * the same name without the suffix. */
rq_status rmsnorm_quant_fp8_per_token_f16(
    const uint16_t* x, int64_t ldx, const uint16_t* residual, int64_t ldr,
    const uint16_t* weight, int64_t M, int64_t H, float eps,
    uint16_t* residual_out, uint8_t* q_out, float* scale_out, uint16_t* y_out,
    void* stream);
rq_status rmsnorm_quant_fp8_per_group_f16(
    const uint16_t* x, int64_t ldx, const uint16_t* residual, int64_t ldr,
    const uint16_t* weight, int64_t M, int64_t H, float eps, int64_t group,
    uint16_t* residual_out, uint8_t* q_out, float* scale_out, uint16_t* y_out,
    void* stream);
rq_status rmsnorm_quant_mxfp4_f16(
    const uint16_t* x, int64_t ldx, const uint16_t* residual, int64_t ldr,
    const uint16_t* weight, int64_t M, int64_t H, float eps,
    uint16_t* residual_out, uint8_t* q_out, uint8_t* scale_out, uint16_t* y_out,
    void* stream);
rq_status rmsnorm_residual_f16(
    const uint16_t* x, int64_t ldx, const uint16_t* residual, int64_t ldr,
    const uint16_t* weight, int64_t M, int64_t H, float eps,
    uint16_t* residual_out, uint16_t* y_out, void* stream);
rq_status quantize_fp8_per_token_f16(
    const uint16_t* y, int64_t ldy, int64_t M, int64_t H,
    uint8_t* q_out, float* scale_out, void* stream);
rq_status quantize_fp8_per_group_f16(
    const uint16_t* y, int64_t ldy, int64_t M, int64_t H, int64_t group,
    uint8_t* q_out, float* scale_out, void* stream);
rq_status quantize_mxfp4_f16(
    const uint16_t* y, int64_t ldy, int64_t M, int64_t H,
    uint8_t* q_out, uint8_t* scale_out, void* stream);

/* ---- column-major scales ----
 * The review of sglang PR #29723 names a transpose of the activation scales
 * for the GEMM that takes preshuffled weights (_maybe_transpose_aiter_
 * bpreshuffle_scale) without stating the layout.  Read here as: the scales
 * stored column-major, one contiguous run of M values per group or block,
 * with a leading dimension the caller may pad.  The values are exactly those
 * of the row-major calls; only where they are stored differs:
 *  scale_out  per-group FP8: fp32 [H / group, ld_scale], scale of row m and
 *             group g at scale_out[g * ld_scale + m];
 *             MXFP4: uint8 E8M0 [H / 32, ld_scale], same indexing
 *  ld_scale   >= max(M, 1); entries past M in each run are not written
 * Everything else (arguments, layouts of the other outputs, aliasing, errors)
 * as rmsnorm_quant_fp8_per_group / rmsnorm_quant_mxfp4; ld_scale < 1 or
 * < M is RQ_ERR_INVALID.  The _f16 names take fp16 rows. */
rq_status rmsnorm_quant_fp8_per_group_tscale(
    const uint16_t* x, int64_t ldx, const uint16_t* residual, int64_t ldr,
    const uint16_t* weight, int64_t M, int64_t H, float eps, int64_t group,
    uint16_t* residual_out, uint8_t* q_out, float* scale_out, int64_t ld_scale,
    uint16_t* y_out, void* stream);
rq_status rmsnorm_quant_mxfp4_tscale(
    const uint16_t* x, int64_t ldx, const uint16_t* residual, int64_t ldr,
    const uint16_t* weight, int64_t M, int64_t H, float eps,
    uint16_t* residual_out, uint8_t* q_out, uint8_t* scale_out, int64_t ld_scale,
    uint16_t* y_out, void* stream);
rq_status rmsnorm_quant_fp8_per_group_tscale_f16(
    const uint16_t* x, int64_t ldx, const uint16_t* residual, int64_t ldr,
    const uint16_t* weight, int64_t M, int64_t H, float eps, int64_t group,
    uint16_t* residual_out, uint8_t* q_out, float* scale_out, int64_t ld_scale,
    uint16_t* y_out, void* stream);
rq_status rmsnorm_quant_mxfp4_tscale_f16(
    const uint16_t* x, int64_t ldx, const uint16_t* residual, int64_t ldr,
    const uint16_t* weight, int64_t M, int64_t H, float eps,
    uint16_t* residual_out, uint8_t* q_out, uint8_t* scale_out, int64_t ld_scale,
    uint16_t* y_out, void* stream);

/* QK GemmaRMSNorm + gate de-interleave.  sglang PR #27656 ("Fuse QK RMSNorm +
 * gate extraction Triton kernel for Qwen3.5 on HIP"), Motivation and
 * Modifications: reads q and gate from the interleaved per-token layout
 * [q_h0 | gate_h0 | q_h1 | gate_h1 | ...], applies GemmaRMSNorm
 * (v * rstd * (1 + w)) to every head of q and k, writes contiguous q, k and
 * gate; the review asks for k to be read through its stride, not copied.
 *
 *  qg        [T, ld_qg] bf16, ld_qg >= 2 * Hq * D; head h of token t has q at
 *            columns [2Dh, 2Dh + D) and gate at [2Dh + D, 2D(h + 1))
 *  k         [T, ld_k] bf16, ld_k >= Hk * D; head h at columns [Dh, D(h + 1))
 *  q_w, k_w  [D] bf16 weights, applied as (1 + w)
 *  D         head dimension: a multiple of 8, at most RQ_MAX_HEAD_DIM
 *  Hq, Hk    heads per token, each at most 65536
 *  q_out     [T, Hq, D] bf16 out; k_out [T, Hk, D]; gate_out [T, Hq, D]
 *            (gate is copied bit for bit)
 */
rq_status qk_gemma_rmsnorm_gate(
    const uint16_t* qg, int64_t ld_qg, const uint16_t* k, int64_t ld_k,
    const uint16_t* q_w, const uint16_t* k_w, int64_t T, int64_t Hq, int64_t Hk,
    int64_t D, float eps, uint16_t* q_out, uint16_t* k_out, uint16_t* gate_out,
    void* stream);

/* QK GemmaRMSNorm + gate de-interleave with FP8 q and k.  The step above,
 * followed by the downstream quantization of the attention inputs that the
 * pages fuse elsewhere into the step before a quantized consumer (sglang PR
 * #29723, Motivation; sgl-amd-mono PR #26 commit notes on the FP8 copy of the
 * next attention input).  Each normalized bf16 head (bit-identical to what
 * qk_gemma_rmsnorm_gate writes) is one granule of the per-token FP8 rule:
 * scale = amax / 448 (fp32, IEEE-equal), codes = E4M3FN(v / scale), nearest
 * even, saturating; an all-zero head has scale 0 and codes +-0.
 *
 *  qg, k, q_w, k_w, T, Hq, Hk, D, eps   as for qk_gemma_rmsnorm_gate
 *  q_codes   [T, Hq, D] uint8 out: E4M3FN codes (8-byte aligned)
 *  q_scale   [T, Hq] fp32 out: one scale per head of each token
 *  k_codes   [T, Hk, D] uint8 out; k_scale [T, Hk] fp32 out
 *  gate_out  [T, Hq, D] bf16 out (copied bit for bit)
 * Errors as for qk_gemma_rmsnorm_gate; a null or misaligned scale pointer is
 * RQ_ERR_INVALID / RQ_ERR_UNSUPPORTED, and scales may not overlap any other
 * buffer.
 */
rq_status qk_gemma_rmsnorm_gate_fp8(
    const uint16_t* qg, int64_t ld_qg, const uint16_t* k, int64_t ld_k,
    const uint16_t* q_w, const uint16_t* k_w, int64_t T, int64_t Hq, int64_t Hk,
    int64_t D, float eps, uint8_t* q_codes, float* q_scale, uint8_t* k_codes,
    float* k_scale, uint16_t* gate_out, void* stream);

/* QK GemmaRMSNorm + gate de-interleave with MXFP4 q and k: each normalized
 * bf16 head (bit-identical to what qk_gemma_rmsnorm_gate writes) is
 * quantized as an MXFP4 row of D values, exactly as rmsnorm_quant_mxfp4
 * quantizes y (one E8M0 byte per 32 elements, E2M1 codes two per byte).
 *
 *  qg, k, q_w, k_w, T, Hq, Hk, eps   as for qk_gemma_rmsnorm_gate
 *  D         a multiple of 32, at most RQ_MAX_HEAD_DIM (else RQ_ERR_UNSUPPORTED)
 *  q_codes   [T, Hq, D / 2] uint8 out (4-byte aligned): element 2j of a head
 *            in the low nibble of byte j
 *  q_scale   [T, Hq, D / 32] uint8 out: E8M0 bytes
 *  k_codes   [T, Hk, D / 2] uint8 out; k_scale [T, Hk, D / 32] uint8 out
 *  gate_out  [T, Hq, D] bf16 out (copied bit for bit)
 * Errors as for qk_gemma_rmsnorm_gate_fp8. */
rq_status qk_gemma_rmsnorm_gate_mxfp4(
    const uint16_t* qg, int64_t ld_qg, const uint16_t* k, int64_t ld_k,
    const uint16_t* q_w, const uint16_t* k_w, int64_t T, int64_t Hq, int64_t Hk,
    int64_t D, float eps, uint8_t* q_codes, uint8_t* q_scale, uint8_t* k_codes,
    uint8_t* k_scale, uint16_t* gate_out, void* stream);

/* Static, human-readable name of a status code. */
const char* rq_status_string(rq_status status);

#ifdef __cplusplus
}
#endif

#endif /* RMSNORM_QUANT_H */
