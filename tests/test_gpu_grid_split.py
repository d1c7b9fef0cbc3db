"""Batches split over several launches, reached with small batches.

The library enqueues a batch whose grid would pass 2^31 work-items as several
launches of the same kernel, each told its first row (row kernels) or first
token (QK kernels).  The QK split needs about 16 GB of heads at the real limit,
so it is exercised here through a build of the same source with the limit
lowered to 2^14 work-items (librmsnorm_quant_gridsplit.so, built by build()):
a few hundred rows or tokens then take several launches.  Every output must be
bit-identical to the single-launch call of the main library, and match the
oracle to the usual bar."""

from contextlib import contextmanager

import numpy as np
import pytest
import torch

import rmsnorm_activation_quantization_amd as rq
from parity import check_bf16_close, check_fp8, check_mxfp4, to_np
from rmsnorm_activation_quantization_amd import _build, binding, inputs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
LIMIT = 16384


@pytest.fixture(scope="module")
def split_lib():
    return binding.load(_build.GRID_SPLIT_LIBRARY)


@contextmanager
def using(handle):
    """Run the binding's calls against another build of the library."""
    old = binding._lib
    binding._lib = handle
    binding._FN_CACHE.clear()
    try:
        yield
    finally:
        binding._lib = old
        binding._FN_CACHE.clear()


def launches_rows(M, H):
    lanes = 64 * {256: 1, 4096: 8, 7168: 16}[H]
    return -(-M // (LIMIT // lanes))


def same(a, b):
    for u, v in zip(a, b):
        if u is None:
            assert v is None
            continue
        assert torch.equal(u.contiguous().view(torch.uint8), v.contiguous().view(torch.uint8))


ROW_CASES = [(300, 4096, torch.bfloat16), (100, 7168, torch.bfloat16), (1000, 256, torch.bfloat16),
             (300, 4096, torch.float16)]


@pytest.mark.parametrize("M,H,dt", ROW_CASES)
@pytest.mark.parametrize("fmt", ["fp8_token", "fp8_group", "mxfp4"])
def test_rows_split(ref, split_lib, M, H, dt, fmt):
    assert launches_rows(M, H) >= 4
    d = inputs.random_rows(M, H, 9000 + M, dtype=dt)
    x, r, w = (d[k].to(DEV) for k in ("x", "residual", "weight"))
    fn = {"fp8_token": rq.rmsnorm_quant_fp8_per_token, "fp8_group": rq.rmsnorm_quant_fp8_per_group,
          "mxfp4": rq.rmsnorm_quant_mxfp4}[fmt]
    extra = (128,) if fmt == "fp8_group" else ()
    one = fn(x, r, w, 1e-6, *extra, emit_y=True)
    with using(split_lib):
        many = fn(x, r, w, 1e-6, *extra, emit_y=True)
    torch.cuda.synchronize()
    same(one, many)
    q, ro, sc, y = many
    gpu = to_np(dict(q=q, residual_out=ro, scale=sc, y=y))
    xb, rb, wb = (inputs.bits(d[k]) for k in ("x", "residual", "weight"))
    kind = "fp16" if dt == torch.float16 else "bf16"
    if fmt == "mxfp4":
        o = ref.mxfp4(xb, rb, wb, 1e-6, emit_y=True, dtype=kind)
        check_mxfp4(gpu, o, ref.quantize_mxfp4(gpu["y"], dtype=kind), f"split {fmt} [{M}, {H}]")
    else:
        g = H if fmt == "fp8_token" else 128
        o = (ref.fp8_per_token(xb, rb, wb, 1e-6, emit_y=True, dtype=kind) if fmt == "fp8_token"
             else ref.fp8_per_group(xb, rb, wb, 1e-6, 128, emit_y=True, dtype=kind))
        check_fp8(gpu, o, ref.quantize_fp8(gpu["y"], g, dtype=kind), g, f"split {fmt} [{M}, {H}]")


@pytest.mark.parametrize("M", [300, 1501])
def test_tscale_and_unfused_split(split_lib, M):
    """Both sizes take rows of 8 waves with one chunk a lane.  [300, 4096]
    stores its column-major scales directly; [1501, 4096] stages them, and
    column-major MXFP4 takes two rows in turn a workgroup.  Under the lowered
    limit a launch holds 32 rows: [1501, 4096] takes 47 launches, the last of
    29 rows, whose last workgroup's second turn is past the end."""
    H = 4096
    d = inputs.random_rows(M, H, 9100 + M)
    x, r, w = (d[k].to(DEV) for k in ("x", "residual", "weight"))
    calls = [lambda: rq.rmsnorm_quant_mxfp4_tscale(x, r, w, 1e-6),
             lambda: rq.rmsnorm_quant_fp8_per_group_tscale(x, r, w, 1e-6, 128),
             lambda: rq.rmsnorm_residual_bf16(x, r, w, 1e-6),
             lambda: rq.quantize_mxfp4(x), lambda: rq.quantize_fp8_per_token(x)]
    for c in calls:
        one = c()
        with using(split_lib):
            many = c()
        torch.cuda.synchronize()
        same(one, many)


QK_CASES = [(100, 16, 2, 256), (400, 8, 1, 128), (100, 4, 4, 512)]


@pytest.mark.parametrize("T,Hq,Hk,D", QK_CASES)
def test_qk_split(ref, split_lib, T, Hq, Hk, D):
    heads_per_wave = 64 // max(1, D // 8)
    tokens_per_launch = LIMIT // 64 * heads_per_wave // (Hq + Hk)
    assert -(-T // tokens_per_launch) >= 3
    w = inputs.QKWorkload("qk_split", T, Hq, Hk, D, seed=9200 + T)
    d = inputs.qk_inputs(w)
    dev_in = [d[n].to(DEV) for n in ("qg", "k", "q_w", "k_w")]
    outs = {}
    for name, fn in (("bf16", rq.qk_gemma_rmsnorm_gate), ("fp8", rq.qk_gemma_rmsnorm_gate_fp8),
                     ("mxfp4", rq.qk_gemma_rmsnorm_gate_mxfp4)):
        one = fn(*dev_in, Hq, Hk, D, w.eps)
        with using(split_lib):
            many = fn(*dev_in, Hq, Hk, D, w.eps)
        torch.cuda.synchronize()
        same(one, many)
        outs[name] = many
    host = [inputs.bits(d[n]) for n in ("qg", "k", "q_w", "k_w")]
    o = ref.qk_gemma_rmsnorm_gate(*host, Hq, Hk, D, w.eps)
    q, k, gate = outs["bf16"]
    assert (inputs.bits(gate) == o["gate"]).all()
    check_bf16_close(inputs.bits(q), o["q"], "split q")
    check_bf16_close(inputs.bits(k), o["k"], "split k")
    # the quantized heads are the quantization of the bf16 heads just checked
    q8, qs8, k8, ks8, _ = outs["fp8"]
    want = ref.quantize_fp8(inputs.bits(q).reshape(-1, D), D)
    assert (q8.view(torch.uint8).cpu().numpy().reshape(-1, D) == want["q"]).all()
    assert np.array_equal(qs8.cpu().numpy().reshape(-1).view(np.uint32), want["scale"].reshape(-1).view(np.uint32))
    q4, qs4, k4, ks4, _ = outs["mxfp4"]
    want = ref.quantize_mxfp4(inputs.bits(k).reshape(-1, D))
    assert (k4.cpu().numpy().reshape(-1, D // 2) == want["q"]).all()
    assert (ks4.cpu().numpy().reshape(-1, D // 32) == want["scale"]).all()
