"""MI355X (gfx950) fused residual-add -> RMSNorm -> activation quantization.

The compute lives in librmsnorm_quant.so (hand-written HIP kernels behind a C
ABI, include/rmsnorm_quant.h); this package only marshals torch tensors into
that ABI.  Entry points keep the C names:

  rmsnorm_quant_fp8_per_token   residual add + RMSNorm + per-token FP8 E4M3FN
  rmsnorm_quant_fp8_per_group   ... + per-group FP8 (group 32..512)
  rmsnorm_quant_mxfp4           ... + MXFP4 (E2M1 codes, E8M0 scale per 32)
  rmsnorm_quant_fp8_per_group_tscale / rmsnorm_quant_mxfp4_tscale
                                the same with column-major scales [groups, >= M]
  qk_gemma_rmsnorm_gate         QK GemmaRMSNorm + gate de-interleave
  qk_gemma_rmsnorm_gate_fp8     ... with q and k as FP8 E4M3FN, one scale per head
  qk_gemma_rmsnorm_gate_mxfp4   ... with q and k as MXFP4, one E8M0 scale per 32 elements

and the unfused sequence, one launch per step (bit-identical results):

  rmsnorm_residual_bf16         residual add + RMSNorm -> bf16 y
  quantize_fp8_per_token / quantize_fp8_per_group / quantize_mxfp4

Row functions take bf16 or fp16 tensors and return their rows in the same
dtype (the _f16 names are the same functions, named after the C entry points).
"""

from .binding import (RQ_ERR_DEVICE, RQ_ERR_HIP, RQ_ERR_INVALID, RQ_ERR_UNSUPPORTED, RQ_MAX_HEAD_DIM, RQ_MAX_HIDDEN, RQ_OK,
                      lib, library_path, qk_gemma_rmsnorm_gate, qk_gemma_rmsnorm_gate_fp8, qk_gemma_rmsnorm_gate_mxfp4,
                      quantize_fp8_per_group,
                      rmsnorm_quant_fp8_per_group_tscale, rmsnorm_quant_fp8_per_group_tscale_f16,
                      rmsnorm_quant_mxfp4_tscale, rmsnorm_quant_mxfp4_tscale_f16, quantize_fp8_per_group_f16,
                      quantize_fp8_per_token, quantize_fp8_per_token_f16, quantize_mxfp4, quantize_mxfp4_f16,
                      rmsnorm_quant_fp8_per_group, rmsnorm_quant_fp8_per_group_f16, rmsnorm_quant_fp8_per_token,
                      rmsnorm_quant_fp8_per_token_f16, rmsnorm_quant_mxfp4, rmsnorm_quant_mxfp4_f16,
                      rmsnorm_residual_bf16, rmsnorm_residual_f16, status_string)

__all__ = [
    "rmsnorm_quant_fp8_per_token", "rmsnorm_quant_fp8_per_group", "rmsnorm_quant_mxfp4", "qk_gemma_rmsnorm_gate",
    "qk_gemma_rmsnorm_gate_fp8", "qk_gemma_rmsnorm_gate_mxfp4", "rmsnorm_quant_fp8_per_group_tscale", "rmsnorm_quant_mxfp4_tscale",
    "rmsnorm_quant_fp8_per_group_tscale_f16", "rmsnorm_quant_mxfp4_tscale_f16",
    "rmsnorm_residual_bf16", "quantize_fp8_per_token", "quantize_fp8_per_group", "quantize_mxfp4",
    "rmsnorm_quant_fp8_per_token_f16", "rmsnorm_quant_fp8_per_group_f16", "rmsnorm_quant_mxfp4_f16",
    "rmsnorm_residual_f16", "quantize_fp8_per_token_f16", "quantize_fp8_per_group_f16", "quantize_mxfp4_f16",
    "lib", "library_path", "status_string", "RQ_OK", "RQ_ERR_INVALID", "RQ_ERR_UNSUPPORTED", "RQ_ERR_HIP",
    "RQ_ERR_DEVICE",
    "RQ_MAX_HIDDEN", "RQ_MAX_HEAD_DIM",
]
