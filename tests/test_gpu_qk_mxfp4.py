"""GPU parity of qk_gemma_rmsnorm_gate_mxfp4 (QK GemmaRMSNorm + gate with q and k
quantized to MXFP4, one E8M0 byte per 32 elements of a head) against the CPU oracle.

Checks: the gate is bit-exact; codes and E8M0 bytes are bit-identical to the
oracle's MXFP4 quantization of the bf16 heads that qk_gemma_rmsnorm_gate writes on
the GPU; against the oracle's full result, codes match on at least 99.9 % of
elements and differ by at most one code step, and an E8M0 byte by at most one."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import rmsnorm_activation_quantization_amd as rq
from rmsnorm_activation_quantization_amd import inputs
from parity import CODE_MATCH_MIN, check_bf16_close, code_steps, mxfp4_value_steps
from test_gpu_qk_fp8 import gpu_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def nibbles(packed, D):
    p = packed.reshape(-1, D // 2)
    return np.stack([p & 0xF, p >> 4], axis=-1).reshape(-1, D)


def run(ref, w: inputs.QKWorkload, ld_k=None, ld_qg_pad=0):
    dev_in, host = gpu_inputs(w, ld_k, ld_qg_pad)
    out = rq.qk_gemma_rmsnorm_gate_mxfp4(*dev_in, w.Hq, w.Hk, w.D, w.eps)
    assert out is not None, "a supported QK shape was refused"
    bf = rq.qk_gemma_rmsnorm_gate(*dev_in, w.Hq, w.Hk, w.D, w.eps)
    torch.cuda.synchronize()
    q, qs, k, ks, gate = (t.cpu().numpy() if t.dtype == torch.uint8 else t for t in out)
    qb, kb = inputs.bits(bf[0]), inputs.bits(bf[1])
    o = ref.qk_gemma_rmsnorm_gate_mxfp4(*host, w.Hq, w.Hk, w.D, w.eps)
    ob = ref.qk_gemma_rmsnorm_gate(*host, w.Hq, w.Hk, w.D, w.eps)
    assert (inputs.bits(gate) == o["gate"]).all(), "gate must be a bit-exact copy"
    D = w.D
    for name, codes, scale, heads, H in (("q", q, qs, qb, w.Hq), ("k", k, ks, kb, w.Hk)):
        if w.T * H == 0:
            continue
        req = ref.quantize_mxfp4(heads.reshape(-1, D))
        assert (codes.reshape(-1, D // 2) == req["q"]).all(), f"{w.name} {name}: codes differ from quantize(gpu heads)"
        assert (scale.reshape(-1, D // 32) == req["scale"]).all(), f"{w.name} {name}: E8M0 differ from quantize(gpu heads)"
        g, r = nibbles(codes, D), nibbles(o[name], D)
        match = float((g == r).mean())
        assert match >= CODE_MATCH_MIN, f"{w.name} {name}: only {match:.5f} of codes identical"
        bd = np.abs(scale.reshape(-1).astype(int) - o[name + "_scale"].reshape(-1).astype(int))
        assert bd.max(initial=0) <= 1, f"{w.name} {name}: an E8M0 byte differs by {int(bd.max())}"
        same = np.repeat(bd.reshape(-1, D // 32) == 0, 32, axis=1)
        steps = code_steps(g, r, 0x8)[same]
        assert steps.max(initial=0) <= 1, f"{w.name} {name}: a code is {int(steps.max())} steps off"
        if (~same).any():
            gb = np.repeat(scale.reshape(-1, D // 32).astype(np.int64), 32, axis=1)
            rb = np.repeat(o[name + "_scale"].reshape(-1, D // 32).astype(np.int64), 32, axis=1)
            vs = mxfp4_value_steps(g[~same], gb[~same], r[~same], rb[~same])
            assert vs.max(initial=0) <= 1, f"{w.name} {name}: a code is {vs.max():.2f} coarse steps off"
        if bd.any():
            ga = (heads.reshape(-1, 32).astype(np.int64) & 0x7FFF).max(axis=1)
            oa = (ob[name].reshape(-1, 32).astype(np.int64) & 0x7FFF).max(axis=1)
            assert (np.abs(ga - oa)[bd != 0] == 1).all(), \
                f"{w.name} {name}: an E8M0 byte differs without a one-ulp amax change"
    check_bf16_close(qb, ob["q"], f"{w.name} q heads")
    check_bf16_close(kb, ob["k"], f"{w.name} k heads")


def test_qk_mxfp4_workload(ref):
    run(ref, inputs.QK_DECODE)


def test_qk_mxfp4_strided(ref):
    run(ref, inputs.QK_DECODE, ld_k=1024, ld_qg_pad=64)


@pytest.mark.parametrize("T,Hq,Hk,D", [(1, 1, 1, 32), (3, 4, 1, 64), (5, 8, 2, 128), (7, 2, 2, 512), (9, 3, 0, 256),
                                        (4, 0, 3, 256), (6, 5, 3, 96), (300, 16, 2, 256), (2048, 16, 2, 256)])
def test_qk_mxfp4_shapes(ref, T, Hq, Hk, D):
    run(ref, inputs.QKWorkload(f"qk4_{T}x{Hq}x{Hk}x{D}", T, Hq, Hk, D, seed=5 * T + Hq + D))


def test_qk_mxfp4_tiny_heads_without_eps(ref):
    run(ref, inputs.QKWorkload("qk4_tiny", 8, 4, 2, 128, seed=13, eps=0.0))


def test_qk_mxfp4_closed_forms_and_errors():
    T, Hq, Hk, D = 3, 2, 1, 256
    qg = torch.full((T, 2 * Hq * D), 3.0, dtype=torch.bfloat16, device=DEV)
    k = torch.full((T, Hk * D), -0.25, dtype=torch.bfloat16, device=DEV)
    z = torch.zeros(D, dtype=torch.bfloat16, device=DEV)
    q, qs, kk, ks, gate = rq.qk_gemma_rmsnorm_gate_mxfp4(qg, k, z, z, Hq, Hk, D, 1e-6)
    torch.cuda.synchronize()
    assert (q == 0x66).all() and (kk == 0xEE).all() and (qs == 125).all() and (ks == 125).all()
    assert (gate == 3.0).all()
    # D not a multiple of 32 cannot fuse
    qg = torch.zeros((2, 2 * 40), dtype=torch.bfloat16, device=DEV)
    k = torch.zeros((2, 40), dtype=torch.bfloat16, device=DEV)
    w = torch.zeros(40, dtype=torch.bfloat16, device=DEV)
    assert rq.qk_gemma_rmsnorm_gate_mxfp4(qg, k, w, w, 1, 1, 40, 1e-6) is None
    empty = rq.qk_gemma_rmsnorm_gate_mxfp4(torch.empty((0, 512), dtype=torch.bfloat16, device=DEV),
                                           torch.empty((0, 256), dtype=torch.bfloat16, device=DEV), z, z, 1, 1, D)
    assert empty is not None and empty[0].shape == (0, 1, 128)
