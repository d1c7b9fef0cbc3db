"""The entry points enqueue only kernels, so they can be captured into a HIP
graph: replays (with eager work and synchronizations between them) must
reproduce the eager results bit for bit."""

from __future__ import annotations

import hashlib

import pytest
import torch

import rmsnorm_activation_quantization_amd as rq
from rmsnorm_activation_quantization_amd import inputs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def test_graph_replay_matches_eager():
    d = inputs.row_inputs(inputs.DECODE_4096)
    x, r, w = (d[k].to(DEV) for k in ("x", "residual", "weight"))
    qd = inputs.qk_inputs(inputs.QK_DECODE)
    qg, k, qw, kw = (qd[n].to(DEV) for n in ("qg", "k", "q_w", "k_w"))
    M, H = x.shape
    bufs = dict(
        t=(torch.empty((M, H), dtype=torch.uint8, device=DEV), torch.empty((M, H), dtype=torch.bfloat16, device=DEV),
           torch.empty((M,), dtype=torch.float32, device=DEV)),
        g=(torch.empty((M, H), dtype=torch.uint8, device=DEV), torch.empty((M, H), dtype=torch.bfloat16, device=DEV),
           torch.empty((M, H // 128), dtype=torch.float32, device=DEV)),
        m=(torch.empty((M, H // 2), dtype=torch.uint8, device=DEV),
           torch.empty((M, H), dtype=torch.bfloat16, device=DEV),
           torch.empty((M, H // 32), dtype=torch.uint8, device=DEV)),
    )
    qk_out = (torch.empty((64, 16, 256), dtype=torch.bfloat16, device=DEV),
              torch.empty((64, 2, 256), dtype=torch.bfloat16, device=DEV),
              torch.empty((64, 16, 256), dtype=torch.bfloat16, device=DEV))

    def step():
        q, ro, s = bufs["t"]
        assert rq.rmsnorm_quant_fp8_per_token(x, r, w, 1e-6, q_out=q, residual_out=ro, scale_out=s) is not None
        q, ro, s = bufs["g"]
        assert rq.rmsnorm_quant_fp8_per_group(x, r, w, 1e-6, 128, q_out=q, residual_out=ro, scale_out=s) is not None
        q, ro, s = bufs["m"]
        assert rq.rmsnorm_quant_mxfp4(x, r, w, 1e-6, q_out=q, residual_out=ro, scale_out=s) is not None
        assert rq.qk_gemma_rmsnorm_gate(qg, k, qw, kw, 16, 2, 256, 1e-6, q_out=qk_out[0], k_out=qk_out[1],
                                        gate_out=qk_out[2]) is not None

    def snapshot():
        return [t.clone() for group in bufs.values() for t in group] + [t.clone() for t in qk_out]

    step()
    torch.cuda.synchronize()
    eager = snapshot()

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for i in range(4):
        for t in [t for group in bufs.values() for t in group] + list(qk_out):
            t.zero_()
        _ = (x.float() * 2).sum().item()  # unrelated eager work between replays
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(snapshot(), eager):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), f"replay {i} differs from eager"


def test_graph_replay_unfused_and_fp16():
    """The unfused launches and the fp16 rows inside one captured graph."""
    d = inputs.row_inputs(inputs.DECODE_4096)
    x, r, w = (d[k].to(DEV) for k in ("x", "residual", "weight"))
    d16 = inputs.row_inputs(inputs.DECODE_4096, dtype=torch.float16)
    x16, r16, w16 = (d16[k].to(DEV) for k in ("x", "residual", "weight"))
    M, H = x.shape
    ro, y = torch.empty_like(x), torch.empty_like(x)
    q = torch.empty((M, H), dtype=torch.uint8, device=DEV)
    s = torch.empty((M,), dtype=torch.float32, device=DEV)
    ro16 = torch.empty_like(x16)
    q16 = torch.empty((M, H // 2), dtype=torch.uint8, device=DEV)
    s16 = torch.empty((M, H // 32), dtype=torch.uint8, device=DEV)
    bufs = [ro, y, q, s, ro16, q16, s16]

    def step():
        assert rq.rmsnorm_residual_bf16(x, r, w, 1e-6, residual_out=ro, y_out=y) is not None
        assert rq.quantize_fp8_per_token(y, q_out=q, scale_out=s) is not None
        assert rq.rmsnorm_quant_mxfp4(x16, r16, w16, 1e-6, residual_out=ro16, q_out=q16, scale_out=s16) is not None

    step()
    torch.cuda.synchronize()
    eager = [t.clone() for t in bufs]
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        step()
    torch.cuda.current_stream().wait_stream(st)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for i in range(3):
        for t in bufs:
            t.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(bufs, eager):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), f"replay {i} differs from eager"


def test_graph_replay_stress_bitwise():
    """3000 replays of a captured decode graph (per-group FP8, MXFP4 with
    column-major scales, QK-FP8), the outputs hashed (SHA-256) every 100
    replays and compared with the eager result's hash; a one-bit change of a
    copy must change the hash (positive control of the comparison itself)."""
    d = inputs.row_inputs(inputs.FP8_GROUP_DECODE)
    x, r, w = (d[k].to(DEV) for k in ("x", "residual", "weight"))
    qd = inputs.qk_inputs(inputs.QK_DECODE)
    qg, k, qw, kw = (qd[n].to(DEV) for n in ("qg", "k", "q_w", "k_w"))
    M, H = x.shape
    q8, ro8, s8 = (torch.empty((M, H), dtype=torch.uint8, device=DEV), torch.empty_like(x),
                   torch.empty((M, H // 128), dtype=torch.float32, device=DEV))
    q4, ro4, s4 = (torch.empty((M, H // 2), dtype=torch.uint8, device=DEV), torch.empty_like(x),
                   torch.empty((H // 32, M), dtype=torch.uint8, device=DEV))
    qc = (torch.empty((64, 16, 256), dtype=torch.uint8, device=DEV), torch.empty((64, 16), device=DEV),
          torch.empty((64, 2, 256), dtype=torch.uint8, device=DEV), torch.empty((64, 2), device=DEV),
          torch.empty((64, 16, 256), dtype=torch.bfloat16, device=DEV))
    outs = [q8, ro8, s8, q4, ro4, s4, *qc]

    def step():
        assert rq.rmsnorm_quant_fp8_per_group(x, r, w, 1e-6, 128, q_out=q8, residual_out=ro8, scale_out=s8) is not None
        assert rq.rmsnorm_quant_mxfp4_tscale(x, r, w, 1e-6, q_out=q4, residual_out=ro4, scale_out=s4) is not None
        assert rq.qk_gemma_rmsnorm_gate_fp8(qg, k, qw, kw, 16, 2, 256, 1e-6, q_out=qc[0], q_scale_out=qc[1],
                                            k_out=qc[2], k_scale_out=qc[3], gate_out=qc[4]) is not None

    def digest(tensors):
        h = hashlib.sha256()
        for t in tensors:
            h.update(t.contiguous().view(torch.uint8).cpu().numpy().tobytes())
        return h.hexdigest()

    step()
    torch.cuda.synchronize()
    want = digest(outs)
    flipped = [t.clone() for t in outs]
    flipped[3].view(torch.uint8).view(-1)[7] ^= 1
    assert digest(flipped) != want, "the hash comparison must see a one-bit change"

    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        step()
    torch.cuda.current_stream().wait_stream(st)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for i in range(30):
        for t in outs:
            t.zero_()
        for _ in range(100):
            g.replay()
        torch.cuda.synchronize()
        assert digest(outs) == want, f"outputs differ from the eager result after {100 * (i + 1)} replays"


def test_graph_replay_quantized_qk_and_column_major_scales():
    """The QK entry points with FP8 and MXFP4 q and k, and the column-major-scale
    row calls, inside one captured graph; each replay reproduces the eager
    results bit for bit (outputs cleared by fill kernels between replays)."""
    d = inputs.row_inputs(inputs.DECODE_4096)
    x, r, w = (d[k].to(DEV) for k in ("x", "residual", "weight"))
    qd = inputs.qk_inputs(inputs.QK_DECODE)
    qg, k, qw, kw = (qd[n].to(DEV) for n in ("qg", "k", "q_w", "k_w"))
    M, H = x.shape
    u8, f32, bf = torch.uint8, torch.float32, torch.bfloat16
    outs = dict(
        q8=torch.empty((64, 16, 256), dtype=u8, device=DEV), qs8=torch.empty((64, 16), dtype=f32, device=DEV),
        k8=torch.empty((64, 2, 256), dtype=u8, device=DEV), ks8=torch.empty((64, 2), dtype=f32, device=DEV),
        g8=torch.empty((64, 16, 256), dtype=bf, device=DEV),
        q4=torch.empty((64, 16, 128), dtype=u8, device=DEV), qs4=torch.empty((64, 16, 8), dtype=u8, device=DEV),
        k4=torch.empty((64, 2, 128), dtype=u8, device=DEV), ks4=torch.empty((64, 2, 8), dtype=u8, device=DEV),
        g4=torch.empty((64, 16, 256), dtype=bf, device=DEV),
        tq=torch.empty((M, H), dtype=u8, device=DEV), tro=torch.empty((M, H), dtype=bf, device=DEV),
        ts=torch.empty((H // 128, M + 8), dtype=f32, device=DEV),
        mq=torch.empty((M, H // 2), dtype=u8, device=DEV), mro=torch.empty((M, H), dtype=bf, device=DEV),
        ms=torch.empty((H // 32, M + 8), dtype=u8, device=DEV),
    )

    def step():
        o = outs
        assert rq.qk_gemma_rmsnorm_gate_fp8(qg, k, qw, kw, 16, 2, 256, 1e-6, q_out=o["q8"], q_scale_out=o["qs8"],
                                            k_out=o["k8"], k_scale_out=o["ks8"], gate_out=o["g8"]) is not None
        assert rq.qk_gemma_rmsnorm_gate_mxfp4(qg, k, qw, kw, 16, 2, 256, 1e-6, q_out=o["q4"], q_scale_out=o["qs4"],
                                              k_out=o["k4"], k_scale_out=o["ks4"], gate_out=o["g4"]) is not None
        assert rq.rmsnorm_quant_fp8_per_group_tscale(x, r, w, 1e-6, 128, q_out=o["tq"], residual_out=o["tro"],
                                                     scale_out=o["ts"][:, :M]) is not None
        assert rq.rmsnorm_quant_mxfp4_tscale(x, r, w, 1e-6, q_out=o["mq"], residual_out=o["mro"],
                                             scale_out=o["ms"][:, :M]) is not None

    def snapshot():
        return [t.clone() for t in outs.values()]

    for t in outs.values():
        t.zero_()
    step()
    torch.cuda.synchronize()
    eager = snapshot()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for i in range(4):
        for t in outs.values():
            t.zero_()
        _ = (x.float() * 3).sum().item()
        g.replay()
        torch.cuda.synchronize()
        for name, a, b in zip(outs, snapshot(), eager):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), f"replay {i}: {name} differs from eager"


def test_graph_replay_staged_column_major_scales():
    """Batches large enough for the staged column-major kernels (scales run
    along M through LDS, MXFP4 rows two in turn a workgroup): [1101, 4096], an
    odd count, so the last MXFP4 workgroup's second turn is past the end.  Each
    replay reproduces the eager results bit for bit, padding past M untouched."""
    M, H = 1101, 4096
    d = inputs.random_rows(M, H, seed=1101)
    x, r, w = (d[k].to(DEV) for k in ("x", "residual", "weight"))
    u8, f32, bf = torch.uint8, torch.float32, torch.bfloat16
    outs = dict(
        tq=torch.empty((M, H), dtype=u8, device=DEV), tro=torch.empty((M, H), dtype=bf, device=DEV),
        ts=torch.empty((H // 128, M + 3), dtype=f32, device=DEV),
        mq=torch.empty((M, H // 2), dtype=u8, device=DEV), mro=torch.empty((M, H), dtype=bf, device=DEV),
        ms=torch.empty((H // 32, M + 3), dtype=u8, device=DEV),
    )

    def step():
        o = outs
        assert rq.rmsnorm_quant_fp8_per_group_tscale(x, r, w, 1e-6, 128, q_out=o["tq"], residual_out=o["tro"],
                                                     scale_out=o["ts"][:, :M]) is not None
        assert rq.rmsnorm_quant_mxfp4_tscale(x, r, w, 1e-6, q_out=o["mq"], residual_out=o["mro"],
                                             scale_out=o["ms"][:, :M]) is not None

    def snapshot():
        return [t.clone() for t in outs.values()]

    for t in outs.values():
        t.zero_()
    step()
    torch.cuda.synchronize()
    eager = snapshot()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for i in range(4):
        for t in outs.values():
            t.zero_()
        _ = (x.float() * 3).sum().item()
        g.replay()
        torch.cuda.synchronize()
        for name, a, b in zip(outs, snapshot(), eager):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), f"replay {i}: {name} differs from eager"
        assert (outs["ts"][:, M:] == 0).all() and (outs["ms"][:, M:] == 0).all(), "padding past M written"
