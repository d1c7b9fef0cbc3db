"""Host-side argument checks of the Python binding (no GPU: every case is
refused before the library is called)."""

import os

import pytest
import torch

import rmsnorm_activation_quantization_amd as rq


@pytest.fixture(scope="module", autouse=True)
def built():
    """The checks run in the marshalling module, which the binding calls with
    entry points of the loaded library: build both if a fresh checkout has
    neither (the HIP library cross-compiles without a GPU)."""
    from rmsnorm_activation_quantization_amd import _build
    if not os.path.exists(_build.LIBRARY):
        _build.build()
    if not os.path.exists(_build.marshal_path()):
        _build.build_marshal()


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


def test_missing_library_fails_loudly(monkeypatch):
    """No other code path: without the built library every call raises."""
    from rmsnorm_activation_quantization_amd import binding
    monkeypatch.setattr(binding, "_lib", None)
    monkeypatch.setattr(binding._build, "LIBRARY", "/nonexistent/librmsnorm_quant.so")
    monkeypatch.setattr(binding, "_FN_CACHE", {})
    with pytest.raises(RuntimeError, match="missing"):
        binding.lib()
    with pytest.raises(RuntimeError, match="missing"):
        rq.rmsnorm_quant_mxfp4(*rows())


def test_missing_marshalling_module_fails_loudly(monkeypatch):
    """No other code path: without the built marshalling module every call raises."""
    import sys
    from rmsnorm_activation_quantization_amd import binding
    import rmsnorm_activation_quantization_amd as pkg
    monkeypatch.setattr(binding, "_marshal", None)
    monkeypatch.delattr(pkg, "_marshal", raising=False)  # else the import finds the loaded module on the package
    monkeypatch.setitem(sys.modules, "rmsnorm_activation_quantization_amd._marshal", None)
    with pytest.raises(RuntimeError, match="missing or does not load"):
        rq.quantize_mxfp4(torch.zeros(4, 256, dtype=torch.bfloat16))


def test_entry_point_addresses():
    """The marshalling module calls the entry points the binding resolves from
    the loaded library: the bf16 and fp16 row functions (the norm launch's
    bf16 one under its _bf16 name), and the QK functions."""
    import ctypes
    from rmsnorm_activation_quantization_amd import binding
    h = binding.lib()
    addr = lambda f: ctypes.cast(f, ctypes.c_void_p).value
    assert binding._entries("rmsnorm_quant_mxfp4") == (addr(h.rmsnorm_quant_mxfp4), addr(h.rmsnorm_quant_mxfp4_f16))
    assert binding._entries("rmsnorm_residual") == (addr(h.rmsnorm_residual_bf16), addr(h.rmsnorm_residual_f16))
    assert binding._entry("qk_gemma_rmsnorm_gate_fp8") == addr(h.qk_gemma_rmsnorm_gate_fp8)
    assert len(set(binding._entries("quantize_fp8_per_group"))) == 2


def test_status_mapping():
    """'Cannot fuse' (a shape or alignment the kernels do not take) is the
    binding's None; a device that is not an MI355X, a failed launch and an
    unknown code raise, and so does an invalid argument."""
    from rmsnorm_activation_quantization_amd import binding
    assert binding._check(rq.RQ_OK, "f") is True
    assert binding._check(rq.RQ_ERR_UNSUPPORTED, "f") is False
    with pytest.raises(ValueError):
        binding._check(rq.RQ_ERR_INVALID, "f")
    with pytest.raises(RuntimeError, match="gfx950"):
        binding._check(rq.RQ_ERR_DEVICE, "f")
    with pytest.raises(RuntimeError):
        binding._check(rq.RQ_ERR_HIP, "f")
    with pytest.raises(RuntimeError):
        binding._check(99, "f")
