"""Host-side argument checks of the Python binding (no GPU: every case is
refused before the library is called)."""

import pytest
import torch

import rmsnorm_activation_quantization_amd as rq


def rows(M=4, H=256, dtype=torch.bfloat16):
    return torch.zeros(M, H, dtype=dtype), torch.zeros(M, H, dtype=dtype), torch.ones(H, dtype=dtype)


def test_cpu_tensors_are_refused():
    x, r, w = rows()
    for fn in (rq.rmsnorm_quant_fp8_per_token, rq.rmsnorm_quant_mxfp4, rq.rmsnorm_residual_bf16):
        with pytest.raises(ValueError, match="CUDA"):
            fn(x, r, w)
    with pytest.raises(ValueError, match="CUDA"):
        rq.quantize_fp8_per_token(x)


def test_unsupported_dtypes_are_refused():
    x, r, w = rows(dtype=torch.float32)
    with pytest.raises(ValueError):
        rq.rmsnorm_quant_fp8_per_token(x, r, w)
    with pytest.raises(ValueError):
        rq.quantize_mxfp4(x)


def test_shapes_are_checked():
    with pytest.raises(ValueError):
        rq.rmsnorm_quant_fp8_per_token(torch.zeros(4, 256, 2, dtype=torch.bfloat16), *rows()[1:])
    x = torch.zeros(4, 256, dtype=torch.bfloat16)[:, ::2]  # non-unit column stride
    with pytest.raises(ValueError):
        rq.rmsnorm_quant_fp8_per_token(x, x, torch.ones(128, dtype=torch.bfloat16))


def test_qk_is_bf16_only():
    qg = torch.zeros(4, 512, dtype=torch.float16)
    with pytest.raises(ValueError):
        rq.qk_gemma_rmsnorm_gate(qg, qg, torch.zeros(128, dtype=torch.float16), torch.zeros(128, dtype=torch.float16),
                                 2, 0, 128)


def test_fp16_names_are_the_dispatching_functions():
    assert rq.rmsnorm_quant_fp8_per_token_f16 is rq.rmsnorm_quant_fp8_per_token
    assert rq.rmsnorm_residual_f16 is rq.rmsnorm_residual_bf16
    assert rq.quantize_mxfp4_f16 is rq.quantize_mxfp4


def test_tensors_on_another_device_are_refused():
    from rmsnorm_activation_quantization_amd import binding
    like = torch.zeros(4, 256, dtype=torch.bfloat16)
    binding._same_device(like, a=torch.zeros(3), b=None)
    with pytest.raises(ValueError, match="weight is on meta"):
        binding._same_device(like, weight=torch.empty(256, dtype=torch.bfloat16, device="meta"))


def test_missing_library_fails_loudly(monkeypatch):
    """No other code path: without the built library every call raises."""
    from rmsnorm_activation_quantization_amd import binding
    monkeypatch.setattr(binding, "_lib", None)
    monkeypatch.setattr(binding._build, "LIBRARY", "/nonexistent/librmsnorm_quant.so")
    monkeypatch.setattr(binding, "_FN_CACHE", {})
    with pytest.raises(RuntimeError, match="missing"):
        binding.lib()
    with pytest.raises(RuntimeError, match="missing"):
        binding._fn("rmsnorm_quant_mxfp4", torch.bfloat16)
