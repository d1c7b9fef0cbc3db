"""The binding's argument checks, entry point by entry point: every refused
argument raises ValueError before anything is launched, and the outputs a
caller passes come back as the very same tensors."""

from __future__ import annotations

import types

import pytest
import torch

import rmsnorm_activation_quantization_amd as rq

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
M, H = 8, 1024


def rows(dtype=torch.bfloat16):
    g = torch.Generator(device=DEV).manual_seed(11)
    x = torch.randn(M, H, generator=g, device=DEV).to(dtype)
    r = torch.randn(M, H, generator=g, device=DEV).to(dtype)
    w = torch.randn(H, generator=g, device=DEV).to(dtype)
    return x, r, w


ROW_CALLS = {
    "fp8_token": lambda x, r, w, **kw: rq.rmsnorm_quant_fp8_per_token(x, r, w, 1e-6, **kw),
    "fp8_group": lambda x, r, w, **kw: rq.rmsnorm_quant_fp8_per_group(x, r, w, 1e-6, 128, **kw),
    "mxfp4": lambda x, r, w, **kw: rq.rmsnorm_quant_mxfp4(x, r, w, 1e-6, **kw),
    "fp8_group_tscale": lambda x, r, w, **kw: rq.rmsnorm_quant_fp8_per_group_tscale(x, r, w, 1e-6, 128, **kw),
    "mxfp4_tscale": lambda x, r, w, **kw: rq.rmsnorm_quant_mxfp4_tscale(x, r, w, 1e-6, **kw),
}


@pytest.mark.parametrize("name", sorted(ROW_CALLS))
def test_row_inputs_refused(name):
    fn = ROW_CALLS[name]
    x, r, w = rows()
    with pytest.raises(ValueError, match="2-D"):
        fn(x.view(M, 2, H // 2), r, w)                       # not 2-D
    with pytest.raises(ValueError, match="2-D"):
        fn(x.float(), r, w)                                   # not bf16 / fp16
    with pytest.raises(ValueError, match="dtype of x"):
        fn(x, r.half(), w)                                    # mixed element types
    with pytest.raises(ValueError, match="unit column stride"):
        fn(x, torch.empty(M, 2 * H, dtype=torch.bfloat16, device=DEV)[:, ::2], w)
    with pytest.raises(ValueError, match="residual must be"):
        fn(x, r[:, : H // 2], w)                              # shapes differ
    with pytest.raises(ValueError, match="residual must be"):
        fn(x, r, w[: H // 2])                                 # weight of the wrong length
    with pytest.raises(ValueError, match="weight must be contiguous"):
        fn(x, r, torch.empty(2 * H, dtype=torch.bfloat16, device=DEV)[::2])
    with pytest.raises(ValueError, match="weight is on cpu"):
        fn(x, r, w.cpu())
    with pytest.raises(ValueError, match="residual_out must be"):
        fn(x, r, w, residual_out=torch.empty(M, H + 8, dtype=torch.bfloat16, device=DEV)[:, :H])
    with pytest.raises(ValueError, match="y_out must be"):
        fn(x, r, w, y_out=torch.empty(M, H, dtype=torch.float16, device=DEV))
    with pytest.raises(ValueError, match="stream"):
        fn(x, r, w, stream=object())
    with pytest.raises(ValueError, match="stream must be"):
        fn(x, r, w, stream=types.SimpleNamespace(cuda_stream="s"))  # not an integer handle
    here = torch.cuda.current_stream().cuda_stream
    with pytest.raises(ValueError, match="stream is on cuda:1"):
        fn(x, r, w, stream=types.SimpleNamespace(cuda_stream=here, device_index=1))
    torch.cuda.synchronize()


@pytest.mark.parametrize("name", ["fp8_token", "fp8_group", "mxfp4"])
def test_row_outputs_refused_and_passed_through(name):
    fn = ROW_CALLS[name]
    x, r, w = rows()
    codes = (M, H // 2) if name == "mxfp4" else (M, H)
    scales = {"fp8_token": (M, 1), "fp8_group": (M, H // 128), "mxfp4": (M, H // 32)}[name]
    sdt = torch.uint8 if name == "mxfp4" else torch.float32
    with pytest.raises(ValueError, match="q_out must be"):
        fn(x, r, w, q_out=torch.empty(codes[0], codes[1] + 1, dtype=torch.uint8, device=DEV))
    with pytest.raises(ValueError, match="q_out must be"):
        fn(x, r, w, q_out=torch.empty(codes, dtype=torch.int16, device=DEV))
    with pytest.raises(ValueError, match="q_out must be"):
        fn(x, r, w, q_out=torch.empty(codes, dtype=torch.uint8))  # host memory
    with pytest.raises(ValueError, match="scale_out must be"):
        fn(x, r, w, scale_out=torch.empty(scales[0] + 1, scales[1], dtype=sdt, device=DEV))
    with pytest.raises(ValueError, match="scale_out must be"):
        fn(x, r, w, scale_out=torch.empty(scales, dtype=torch.float16, device=DEV))
    q = torch.empty(codes, dtype=torch.uint8, device=DEV)
    ro = torch.empty(M, H, dtype=torch.bfloat16, device=DEV)
    sc = torch.empty(scales, dtype=sdt, device=DEV)
    y = torch.empty(M, H, dtype=torch.bfloat16, device=DEV)
    out = fn(x, r, w, q_out=q, residual_out=ro, scale_out=sc, y_out=y)
    torch.cuda.synchronize()
    assert out[0].data_ptr() == q.data_ptr() and out[1] is ro and out[2].data_ptr() == sc.data_ptr() and out[3] is y
    if name != "mxfp4":
        assert out[0].dtype == torch.float8_e4m3fn  # a caller's uint8 buffer comes back viewed as FP8
    if name == "fp8_token":  # a [M] scale buffer is accepted and comes back as [M, 1]
        s1 = torch.empty(M, dtype=torch.float32, device=DEV)
        out = fn(x, r, w, scale_out=s1)
        torch.cuda.synchronize()
        assert out[2].shape == (M, 1) and out[2].data_ptr() == s1.data_ptr()


@pytest.mark.parametrize("name", ["fp8_group_tscale", "mxfp4_tscale"])
def test_column_major_scales_refused(name):
    fn = ROW_CALLS[name]
    x, r, w = rows()
    nrows, sdt = (H // 128, torch.float32) if name == "fp8_group_tscale" else (H // 32, torch.uint8)
    with pytest.raises(ValueError, match="unit column stride"):
        fn(x, r, w, scale_out=torch.empty(nrows, M - 1, dtype=sdt, device=DEV))          # fewer columns than rows
    with pytest.raises(ValueError, match="unit column stride"):
        fn(x, r, w, scale_out=torch.empty(nrows + 1, M, dtype=sdt, device=DEV))          # wrong scale count
    with pytest.raises(ValueError, match="unit column stride"):
        fn(x, r, w, scale_out=torch.empty(M, nrows, dtype=sdt, device=DEV).t())          # column stride M
    with pytest.raises(ValueError, match="unit column stride"):
        fn(x, r, w, scale_out=torch.empty(nrows, M, dtype=torch.int32, device=DEV))
    buf = torch.empty(nrows, M + 24, dtype=sdt, device=DEV)
    out = fn(x, r, w, scale_out=buf[:, 3:3 + M + 8])  # a view into a wider buffer: leading dimension M + 24
    torch.cuda.synchronize()
    assert out is not None and out[2].data_ptr() == buf[:, 3:].data_ptr()


@pytest.mark.parametrize("name", ["quantize_fp8_per_token", "quantize_fp8_per_group", "quantize_mxfp4"])
def test_quantize_refused(name):
    fn = getattr(rq, name)
    y = rows()[0]
    with pytest.raises(ValueError, match="2-D"):
        fn(y.float())
    with pytest.raises(ValueError, match="CUDA"):
        fn(y.cpu())
    with pytest.raises(ValueError, match="q_out must be"):
        fn(y, q_out=torch.empty(M + 1, H, dtype=torch.uint8, device=DEV))
    with pytest.raises(ValueError, match="scale_out must be"):
        fn(y, scale_out=torch.empty(M + 1, 64, dtype=torch.float32, device=DEV))


@pytest.mark.parametrize("name", ["qk_gemma_rmsnorm_gate", "qk_gemma_rmsnorm_gate_fp8", "qk_gemma_rmsnorm_gate_mxfp4"])
def test_qk_refused(name):
    fn = getattr(rq, name)
    T, Hq, Hk, D = 4, 2, 1, 64
    qg = torch.zeros(T, 2 * Hq * D, dtype=torch.bfloat16, device=DEV)
    k = torch.zeros(T, Hk * D, dtype=torch.bfloat16, device=DEV)
    wq = torch.zeros(D, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(ValueError, match="same number of tokens"):
        fn(qg, k[: T - 1], wq, wq, Hq, Hk, D)
    with pytest.raises(ValueError, match=r"q_w must be a contiguous \[head_dim\]"):
        fn(qg, k, wq[: D // 2], wq, Hq, Hk, D)
    with pytest.raises(ValueError, match=r"k_w must be a contiguous \[head_dim\]"):
        fn(qg, k, wq, wq.half(), Hq, Hk, D)
    with pytest.raises(ValueError, match="dtype of x"):
        fn(qg.half(), k, wq, wq, Hq, Hk, D)
    # narrower views of wider buffers: the row strides would pass the library's
    # own check, the widths do not
    wide_qg = torch.zeros(T, 4 * Hq * D, dtype=torch.bfloat16, device=DEV)
    wide_k = torch.zeros(T, 4 * Hk * D, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(ValueError, match="columns"):
        fn(wide_qg[:, : 2 * Hq * D - 8], k, wq, wq, Hq, Hk, D)
    with pytest.raises(ValueError, match="columns"):
        fn(qg, wide_k[:, : Hk * D - 8], wq, wq, Hq, Hk, D)
    out = fn(wide_qg[:, : 2 * Hq * D], wide_k[:, : Hk * D], wq, wq, Hq, Hk, D)  # exactly wide enough
    torch.cuda.synchronize()
    assert out is not None
    with pytest.raises(ValueError, match="gate_out"):
        fn(qg, k, wq, wq, Hq, Hk, D, gate_out=torch.empty(T, Hq, D + 1, dtype=torch.bfloat16, device=DEV))
    gate = torch.empty(T, Hq, D, dtype=torch.bfloat16, device=DEV)
    out = fn(qg, k, wq, wq, Hq, Hk, D, gate_out=gate)
    torch.cuda.synchronize()
    assert out is not None and out[-1] is gate
