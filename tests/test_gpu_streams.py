"""The library keeps no state between calls and enqueues only on the stream it
is given: different entry points running at the same time on four streams
(default priority) give the results of the same calls made one after another."""

from __future__ import annotations

import pytest
import torch

import rmsnorm_activation_quantization_amd as rq
from rmsnorm_activation_quantization_amd import inputs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def test_concurrent_streams_match_serial():
    rows = [inputs.random_rows(M, H, seed=M + H) for M, H in ((300, 4096), (16, 7168), (4096, 1024), (8, 2048))]
    dev_rows = [tuple(d[k].to(DEV) for k in ("x", "residual", "weight")) for d in rows]
    qd = inputs.qk_inputs(inputs.QKWorkload("qk_streams", 128, 16, 2, 256, seed=4))
    qk = tuple(qd[n].to(DEV) for n in ("qg", "k", "q_w", "k_w"))

    def calls(stream):
        (x0, r0, w0), (x1, r1, w1), (x2, r2, w2), (x3, r3, w3) = dev_rows
        return [
            lambda: rq.rmsnorm_quant_fp8_per_token(x0, r0, w0, 1e-6, emit_y=True, stream=stream),
            lambda: rq.rmsnorm_quant_mxfp4(x1, r1, w1, 1e-6, stream=stream),
            lambda: rq.rmsnorm_quant_fp8_per_group_tscale(x2, r2, w2, 1e-6, 64, stream=stream),
            lambda: rq.qk_gemma_rmsnorm_gate_fp8(*qk, 16, 2, 256, 1e-6, stream=stream),
            lambda: rq.rmsnorm_quant_fp8_per_group(x3, r3, w3, 1e-6, 128, stream=stream),
        ]

    def flat(outs):
        return [t.view(torch.uint8).clone() for o in outs for t in o if t is not None]

    serial = flat([c() for c in calls(None)])
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(device=DEV) for _ in range(4)]
    for rep in range(3):
        outs = [None] * 5
        for i, c in enumerate(calls(None)):
            s = streams[i % 4]
            with torch.cuda.stream(s):
                outs[i] = calls(s)[i]()
        torch.cuda.synchronize()
        got = flat(outs)
        assert len(got) == len(serial)
        for a, b in zip(got, serial):
            assert torch.equal(a, b), f"repetition {rep}: a concurrent result differs from the serial one"
