"""GPU parity of qk_gemma_rmsnorm_gate_fp8 (QK GemmaRMSNorm + gate with q and k
quantized per head to FP8 E4M3FN) against the CPU oracle.

Checks: the gate is bit-exact; the codes and scales are bit-identical to the
oracle's per-head quantization of the bf16 heads that qk_gemma_rmsnorm_gate
writes on the GPU (the same kernel computes both, so the FP8 variant quantizes
exactly those heads); against the oracle's full result, codes match on at least
99.9 % of elements and differ by at most one code step, and a scale differs only
where the head's largest bf16 value moved by one ulp."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import rmsnorm_activation_quantization_amd as rq
from rmsnorm_activation_quantization_amd import inputs
from oracle_pins import np_bf16_round
from parity import CODE_MATCH_MIN, check_bf16_close, code_steps, signed_key

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def gpu_inputs(w: inputs.QKWorkload, ld_k=None, ld_qg_pad=0):
    d = inputs.qk_inputs(w, ld_k=ld_k)
    qg = d["qg"]
    if ld_qg_pad:
        wide = torch.zeros((w.T, qg.shape[1] + ld_qg_pad), dtype=torch.bfloat16)
        wide[:, : qg.shape[1]] = qg
        qg_dev = wide.to(DEV)[:, : qg.shape[1]]
    else:
        qg_dev = qg.to(DEV)
    k_dev = d["k"].to(DEV)[:, : w.Hk * w.D] if ld_k else d["k"].to(DEV)
    kb = inputs.bits(d["k"])
    host = (inputs.bits(qg), kb[:, :ld_k] if ld_k else kb, inputs.bits(d["q_w"]), inputs.bits(d["k_w"]))
    return (qg_dev, k_dev, d["q_w"].to(DEV), d["k_w"].to(DEV)), host


def check_heads(codes, scale, heads_gpu, o_codes, o_scale, o_heads, what):
    D = codes.shape[-1]
    codes, o_codes = codes.reshape(-1, D), o_codes.reshape(-1, D)
    scale, o_scale = scale.reshape(-1), o_scale.reshape(-1)
    match = float((codes == o_codes).mean()) if codes.size else 1.0
    assert match >= CODE_MATCH_MIN, f"{what}: only {match:.5f} of codes identical"
    nan = ((codes & 0x7F) == 0x7F) | ((o_codes & 0x7F) == 0x7F)
    steps = code_steps(codes, o_codes, 0x80)[~nan]
    assert steps.max(initial=0) <= 1, f"{what}: a code is {int(steps.max())} steps from the oracle's"
    diff = scale.view(np.uint32) != o_scale.view(np.uint32)
    if diff.any():
        ga = np.abs(signed_key(heads_gpu.reshape(-1, D), 0x8000)).max(axis=1)
        oa = np.abs(signed_key(o_heads.reshape(-1, D), 0x8000)).max(axis=1)
        assert (np.abs(ga - oa)[diff] == 1).all(), f"{what}: a scale differs without a one-ulp amax change"
    return match


def run(ref, w: inputs.QKWorkload, ld_k=None, ld_qg_pad=0):
    dev_in, host = gpu_inputs(w, ld_k, ld_qg_pad)
    out = rq.qk_gemma_rmsnorm_gate_fp8(*dev_in, w.Hq, w.Hk, w.D, w.eps)
    assert out is not None, "a supported QK shape was refused"
    bf = rq.qk_gemma_rmsnorm_gate(*dev_in, w.Hq, w.Hk, w.D, w.eps)
    torch.cuda.synchronize()
    q, qs, k, ks, gate = out
    assert q.dtype == torch.float8_e4m3fn and qs.shape == (w.T, w.Hq) and ks.shape == (w.T, w.Hk)
    qc, kc = q.view(torch.uint8).cpu().numpy(), k.view(torch.uint8).cpu().numpy()
    qs, ks = qs.cpu().numpy(), ks.cpu().numpy()
    qb, kb = inputs.bits(bf[0]), inputs.bits(bf[1])
    o = ref.qk_gemma_rmsnorm_gate_fp8(*host, w.Hq, w.Hk, w.D, w.eps)
    ob = ref.qk_gemma_rmsnorm_gate(*host, w.Hq, w.Hk, w.D, w.eps)
    assert (inputs.bits(gate) == o["gate"]).all(), "gate must be a bit-exact copy"
    assert (inputs.bits(bf[2]) == o["gate"]).all()
    # exact: the FP8 heads are the per-head quantization of the GPU's own bf16 heads
    for name, codes, scale, heads, H in (("q", qc, qs, qb, w.Hq), ("k", kc, ks, kb, w.Hk)):
        if w.T * H == 0:
            continue
        req = ref.quantize_fp8(heads.reshape(-1, w.D), w.D)
        assert (codes.reshape(-1, w.D) == req["q"]).all(), f"{w.name} {name}: codes differ from quantize(gpu heads)"
        assert np.array_equal(scale.reshape(-1).view(np.uint32), req["scale"].reshape(-1).view(np.uint32)), \
            f"{w.name} {name}: scales differ from quantize(gpu heads)"
    # tolerance against the oracle's whole result
    check_bf16_close(qb, ob["q"], f"{w.name} q heads")
    check_bf16_close(kb, ob["k"], f"{w.name} k heads")
    mq = check_heads(qc, qs, qb, o["q"], o["q_scale"], ob["q"], f"{w.name} q")
    mk = check_heads(kc, ks, kb, o["k"], o["k_scale"], ob["k"], f"{w.name} k")
    print(f"{w.name}: code match q {mq:.6f} k {mk:.6f}", flush=True)


def test_qk_fp8_workload(ref):
    run(ref, inputs.QK_DECODE)


def test_qk_fp8_strided(ref):
    run(ref, inputs.QK_DECODE, ld_k=1024, ld_qg_pad=64)


@pytest.mark.parametrize("T,Hq,Hk,D", [(1, 1, 1, 8), (3, 4, 1, 64), (5, 8, 2, 128), (7, 2, 2, 512), (9, 3, 0, 256),
                                        (4, 0, 3, 256), (6, 5, 3, 40), (2, 7, 1, 200), (300, 16, 2, 256),
                                        (2048, 16, 2, 256)])
def test_qk_fp8_shapes(ref, T, Hq, Hk, D):
    run(ref, inputs.QKWorkload(f"qk8_{T}x{Hq}x{Hk}x{D}", T, Hq, Hk, D, seed=3 * T + Hq + D))


def test_qk_fp8_tiny_heads_without_eps(ref):
    run(ref, inputs.QKWorkload("qk8_tiny", 8, 4, 2, 128, seed=12, eps=0.0))


def test_qk_fp8_closed_forms():
    """Constant heads with w = 0 normalize to 1 (q) and -1 (k): codes 0x7E / 0xFE,
    scale 1/448.  An all-zero head: scale 0, codes +-0."""
    T, Hq, Hk, D = 3, 2, 1, 256
    qg = torch.full((T, 2 * Hq * D), 3.0, dtype=torch.bfloat16, device=DEV)
    k = torch.full((T, Hk * D), -0.25, dtype=torch.bfloat16, device=DEV)
    z = torch.zeros(D, dtype=torch.bfloat16, device=DEV)
    q, qs, kk, ks, gate = rq.qk_gemma_rmsnorm_gate_fp8(qg, k, z, z, Hq, Hk, D, 1e-6)
    torch.cuda.synchronize()
    assert (q.view(torch.uint8) == 0x7E).all() and (kk.view(torch.uint8) == 0xFE).all()
    inv = np.float32(1.0) / np.float32(448.0)
    assert (qs.cpu().numpy() == inv).all() and (ks.cpu().numpy() == inv).all()
    assert (gate == 3.0).all()
    zq = torch.zeros((1, 2 * D), dtype=torch.bfloat16, device=DEV)
    zk = torch.zeros((1, D), dtype=torch.bfloat16, device=DEV)
    q, qs, kk, ks, _ = rq.qk_gemma_rmsnorm_gate_fp8(zq, zk, z, z, 1, 1, D, 1e-6)
    torch.cuda.synchronize()
    assert (qs == 0).all() and (ks == 0).all()
    assert ((q.view(torch.uint8) & 0x7F) == 0).all() and ((kk.view(torch.uint8) & 0x7F) == 0).all()


def test_qk_fp8_weight_probe():
    """Every value 1024, eps 0: each head is bf16(1 + w); scale = amax / 448 and the
    codes follow from the fp32 quotients, checked here against torch's E4M3FN cast."""
    T, Hq, Hk, D = 2, 2, 1, 256
    qg = torch.full((T, 2 * Hq * D), 1024.0, dtype=torch.bfloat16, device=DEV)
    k = torch.full((T, Hk * D), 1024.0, dtype=torch.bfloat16, device=DEV)
    rng = np.random.default_rng(8)
    qw = inputs.from_bits(np_bf16_round(rng.normal(0, 2.0, D))).to(DEV)
    q, qs, _, _, _ = rq.qk_gemma_rmsnorm_gate_fp8(qg, k, qw, qw, Hq, Hk, D, 0.0)
    torch.cuda.synchronize()
    head = (1.0 + qw.float()).to(torch.bfloat16).float().cpu()
    scale = head.abs().max() / torch.tensor(448.0)
    assert (qs.cpu() == scale).all()
    want = (head / scale).to(torch.float8_e4m3fn).view(torch.uint8)  # |quotient| <= 448: no saturation case
    assert torch.equal(q.view(torch.uint8).cpu()[0, 0], want) and torch.equal(q.view(torch.uint8).cpu()[1, 1], want)


def test_qk_fp8_empty_and_errors():
    D = 128
    w = torch.zeros(D, dtype=torch.bfloat16, device=DEV)
    qg = torch.empty((0, 2 * D), dtype=torch.bfloat16, device=DEV)
    k = torch.empty((0, D), dtype=torch.bfloat16, device=DEV)
    out = rq.qk_gemma_rmsnorm_gate_fp8(qg, k, w, w, 1, 1, D, 1e-6)
    assert out is not None and out[0].shape == (0, 1, D)
    qg = torch.zeros((2, 2 * 520), dtype=torch.bfloat16, device=DEV)   # D above the maximum
    k = torch.zeros((2, 520), dtype=torch.bfloat16, device=DEV)
    w = torch.zeros(520, dtype=torch.bfloat16, device=DEV)
    assert rq.qk_gemma_rmsnorm_gate_fp8(qg, k, w, w, 1, 1, 520, 1e-6) is None
