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


def test_host_threads_through_the_c_abi():
    """Eight host threads call the C entry points at once (ctypes releases the
    interpreter lock, so the calls overlap inside the library), each on its own
    stream with its own buffers, 40 rounds each: every thread's outputs equal
    those of the same calls made one after another on one thread."""
    import threading

    lib = rq.lib()
    n_threads, rounds = 8, 40
    M, H = 16, 7168
    T, Hq, Hk, D = 64, 16, 2, 256
    per = []
    for t in range(n_threads):
        d = inputs.random_rows(M, H, seed=500 + t)
        q = inputs.qk_inputs(inputs.QKWorkload(f"qk_threads_{t}", T, Hq, Hk, D, seed=600 + t))
        per.append(dict(
            x=d["x"].to(DEV), r=d["residual"].to(DEV), w=d["weight"].to(DEV),
            qg=q["qg"].to(DEV), k=q["k"].to(DEV), qw=q["q_w"].to(DEV), kw=q["k_w"].to(DEV),
            ro=torch.empty(M, H, dtype=torch.bfloat16, device=DEV), q8=torch.empty(M, H, dtype=torch.uint8, device=DEV),
            st=torch.empty(M, dtype=torch.float32, device=DEV), q4=torch.empty(M, H // 2, dtype=torch.uint8, device=DEV),
            sm=torch.empty(M, H // 32, dtype=torch.uint8, device=DEV),
            qo=torch.empty(T, Hq, D, dtype=torch.bfloat16, device=DEV), ko=torch.empty(T, Hk, D, dtype=torch.bfloat16, device=DEV),
            go=torch.empty(T, Hq, D, dtype=torch.bfloat16, device=DEV),
            stream=torch.cuda.Stream(device=DEV)))

    def run(p, stream):
        s = stream.cuda_stream if stream is not None else torch.cuda.current_stream().cuda_stream
        st = [lib.rmsnorm_quant_fp8_per_token(p["x"].data_ptr(), H, p["r"].data_ptr(), H, p["w"].data_ptr(), M, H,
                                              1e-6, p["ro"].data_ptr(), p["q8"].data_ptr(), p["st"].data_ptr(), None, s),
              lib.rmsnorm_quant_mxfp4(p["x"].data_ptr(), H, p["r"].data_ptr(), H, p["w"].data_ptr(), M, H, 1e-6,
                                      p["ro"].data_ptr(), p["q4"].data_ptr(), p["sm"].data_ptr(), None, s),
              lib.qk_gemma_rmsnorm_gate(p["qg"].data_ptr(), 2 * Hq * D, p["k"].data_ptr(), Hk * D, p["qw"].data_ptr(),
                                        p["kw"].data_ptr(), T, Hq, Hk, D, 1e-6, p["qo"].data_ptr(), p["ko"].data_ptr(),
                                        p["go"].data_ptr(), s)]
        return st

    keys = ("ro", "q8", "st", "q4", "sm", "qo", "ko", "go")
    serial = []
    for p in per:
        assert run(p, None) == [0, 0, 0]
        torch.cuda.synchronize()
        serial.append({k: p[k].clone() for k in keys})
        for k in keys:
            p[k].zero_()
    torch.cuda.synchronize()

    statuses = [[] for _ in range(n_threads)]

    def worker(i):
        for _ in range(rounds):
            statuses[i].extend(run(per[i], per[i]["stream"]))

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(n_threads)]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    torch.cuda.synchronize()
    for i, p in enumerate(per):
        assert statuses[i] == [0] * (3 * rounds), f"thread {i}: {set(statuses[i])}"
        for k in keys:
            assert torch.equal(p[k].view(torch.uint8), serial[i][k].view(torch.uint8)), f"thread {i}: {k}"
