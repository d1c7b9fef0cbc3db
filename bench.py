"""Benchmark of the fused residual-add -> RMSNorm -> quantization path on one MI355X.

One step = one pass of every step of the hot path over one batch of synthetic
rows resident in HBM:
  rmsnorm_quant_fp8_per_token   [8192, 4096]
  rmsnorm_quant_fp8_per_group   [8192, 4096], group 128
  rmsnorm_quant_mxfp4           [8192, 4096]
  qk_gemma_rmsnorm_gate         64 tokens, 16 q heads, 2 k heads, head dim 256
Consecutive calls read different input sets (4 sets of x and residual rotate,
512 MiB in all, twice the 256 MB Infinity Cache), so every call reads cold rows
from HBM.

value = algorithmic bytes of the step / step time (GB/s).  Algorithmic bytes
count every tensor once: x, residual, weight read; residual_out, codes, scales
written (the optional bf16 side output is not requested here).

The K steps run as one captured HIP graph per kernel (back-to-back launches);
after the W eager warmup steps the graphs are replayed four times untimed (4K
more warmup steps, reported as config.graph_warmup_steps) before the timed
replay.
Also reported: per-kernel time and GB/s in the step (HIP events on the launch
stream) and alone (each prefill kernel's graph replayed in turn, median; the
roofline comes from these), [4096, 4096] in the three formats, decode-size
microseconds per call (M = 16, H = 4096, all formats, C1, C3 and the QK
variants; graph replay of back-to-back calls over rotating inputs, as the
pages time kernels) next to the launch floor of a one-element kernel timed the
same way, and the host time of an eager call through the Python binding; the
unfused sequence, QK and its quantized variants at 8192 tokens,
column-major scales and fp16 rows at [8192, 4096] (each timed alternately with
its bf16 row-major counterpart), and the CPU oracle timed on the host cores as
the CPU baseline.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "achieved HBM GB/s (% of peak) + µs/call at M=16 and M=8192, H=4096"


def row_bytes(fmt: str, M: int, H: int, group: int = 128) -> int:
    base = 2 * M * H * 3 + 2 * H  # x, residual, residual_out, weight
    if fmt == "fp8_token":
        return base + M * H + 4 * M
    if fmt == "fp8_group":
        return base + M * H + 4 * M * (H // group)
    return base + M * H // 2 + M * H // 32


def qk_bytes(T: int, Hq: int, Hk: int, D: int) -> int:
    return 2 * (T * 2 * Hq * D + T * Hk * D + 2 * D) + 2 * (2 * T * Hq * D + T * Hk * D)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--sets", type=int, default=4, help="rotating input sets for the prefill rows")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-decode", action="store_true")
    p.add_argument("--profile-pass", action="store_true",
                   help="short run for rocprofv3: warmup + steps, the prefill kernels alone, the column-major-scale "
                        "calls (4 each at ld = M, then ld = M + 64) and a 256 MiB device copy for calibration")
    p.add_argument("--sweep", action="store_true",
                   help="instead of the step: µs per call and GB/s of the three fused formats and the two "
                        "column-major-scale calls over a range of row counts at H = 4096 and 7168 (one JSON line "
                        "per shape)")
    return p.parse_args()


def sweep(torch, rq, dev, calls: int = 50, replays: int = 5):
    """Row-count sweep of the fused formats, row-major and column-major scales
    (leading dimension M): for each [M, H], a graph of `calls` back-to-back
    calls over rotating input and output sets (at least 512 MiB of inputs, or
    1024 sets), replayed once untimed, then the median replay / calls.
    Inputs ~ N(0, 1), weight ~ N(1, 0.1), drawn on the device from a seeded
    generator."""
    import statistics
    gen = torch.Generator(device=dev).manual_seed(1008)
    for H in (4096, 7168):
        w = (1.0 + 0.1 * torch.randn(H, generator=gen, device=dev)).to(torch.bfloat16)
        for M in (1, 4, 16, 64, 128, 256, 512, 1024, 2048, 4096, 8192):
            n = max(2, min(1024, (512 << 20) // (4 * M * H)))
            xs = torch.randn((n, M, H), generator=gen, device=dev).to(torch.bfloat16)
            rs = torch.randn((n, M, H), generator=gen, device=dev).to(torch.bfloat16)
            no = min(n, 4)
            ro = torch.empty((no, M, H), dtype=torch.bfloat16, device=dev)
            q8 = torch.empty((no, M, H), dtype=torch.uint8, device=dev)
            q4 = torch.empty((no, M, H // 2), dtype=torch.uint8, device=dev)
            st = torch.empty((no, M), dtype=torch.float32, device=dev)
            sg = torch.empty((no, M, H // 128), dtype=torch.float32, device=dev)
            sm = torch.empty((no, M, H // 32), dtype=torch.uint8, device=dev)
            tg = torch.empty((no, H // 128, M), dtype=torch.float32, device=dev)
            tm = torch.empty((no, H // 32, M), dtype=torch.uint8, device=dev)
            fns = {
                "fp8_token": lambda i: rq.rmsnorm_quant_fp8_per_token(
                    xs[i % n], rs[i % n], w, 1e-6, q_out=q8[i % no], residual_out=ro[i % no], scale_out=st[i % no]),
                "fp8_group": lambda i: rq.rmsnorm_quant_fp8_per_group(
                    xs[i % n], rs[i % n], w, 1e-6, 128, q_out=q8[i % no], residual_out=ro[i % no],
                    scale_out=sg[i % no]),
                "mxfp4": lambda i: rq.rmsnorm_quant_mxfp4(
                    xs[i % n], rs[i % n], w, 1e-6, q_out=q4[i % no], residual_out=ro[i % no], scale_out=sm[i % no]),
                "fp8_group_tscale": lambda i: rq.rmsnorm_quant_fp8_per_group_tscale(
                    xs[i % n], rs[i % n], w, 1e-6, 128, q_out=q8[i % no], residual_out=ro[i % no],
                    scale_out=tg[i % no]),
                "mxfp4_tscale": lambda i: rq.rmsnorm_quant_mxfp4_tscale(
                    xs[i % n], rs[i % n], w, 1e-6, q_out=q4[i % no], residual_out=ro[i % no], scale_out=tm[i % no]),
            }
            line = {"M": M, "H": H, "rotating_sets": n}
            for fmt, fn in fns.items():
                for i in range(3):
                    fn(i)
                torch.cuda.synchronize()
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g):
                    for i in range(calls):
                        fn(i)
                upload_graphs(torch, [g], torch.cuda.current_stream())
                g.replay()  # untimed: the first replay after capture runs slower
                torch.cuda.synchronize()
                times = []
                for _ in range(replays):
                    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    a.record()
                    g.replay()
                    b.record()
                    torch.cuda.synchronize()
                    times.append(1000.0 * a.elapsed_time(b) / calls)
                us = statistics.median(times)
                gbs = row_bytes(fmt.replace("_tscale", ""), M, H) / (us * 1e-6) / 1e9
                line[fmt] = {"us": round(us, 3), "GBps": round(gbs, 1), "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4)}
                del g
            print(json.dumps(line), flush=True)
            del xs, rs, ro, q8, q4, st, sg, sm, tg, tm


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for {max(args.gpus, world)}): this path has no multi-GPU "
              "part; its rows shard across GPUs with no communication of their own, and the all-reduce in "
              "front of it is not built here.", file=sys.stderr)
        sys.exit(2)

    import torch

    import rmsnorm_activation_quantization_amd as rq
    from rmsnorm_activation_quantization_amd import inputs

    dev = torch.device("cuda:0")
    rq.lib()
    stream = torch.cuda.current_stream()
    if args.sweep:
        sweep(torch, rq, dev)
        return

    # ---- inputs resident in HBM ----
    wl = inputs.PREFILL
    M, H = wl.M, wl.H
    sets = []
    for s in range(args.sets):
        d = inputs.row_inputs(wl, set_index=s)
        sets.append({k: v.to(dev) for k, v in d.items()})
    outs = []
    for s in range(args.sets):
        outs.append(dict(
            t=(torch.empty((M, H), dtype=torch.uint8, device=dev), torch.empty((M, H), dtype=torch.bfloat16, device=dev),
               torch.empty((M,), dtype=torch.float32, device=dev)),
            g=(torch.empty((M, H), dtype=torch.uint8, device=dev), torch.empty((M, H), dtype=torch.bfloat16, device=dev),
               torch.empty((M, H // 128), dtype=torch.float32, device=dev)),
            m=(torch.empty((M, H // 2), dtype=torch.uint8, device=dev),
               torch.empty((M, H), dtype=torch.bfloat16, device=dev),
               torch.empty((M, H // 32), dtype=torch.uint8, device=dev)),
        ))
    qw = inputs.QK_DECODE
    qd = {k: v.to(dev) for k, v in inputs.qk_inputs(qw).items()}
    # The QK call reads a different copy of its inputs on every call (256 sets of
    # 2.2 MB, 570 MB in all), so that it reads cold rows like the row kernels.
    qk_sets = {n: qd[n].unsqueeze(0).repeat(QK_SETS, 1, 1) for n in ("qg", "k")}
    qk_out = (torch.empty((qw.T, qw.Hq, qw.D), dtype=torch.bfloat16, device=dev),
              torch.empty((qw.T, qw.Hk, qw.D), dtype=torch.bfloat16, device=dev),
              torch.empty((qw.T, qw.Hq, qw.D), dtype=torch.bfloat16, device=dev))

    kernels = ["fp8_token", "fp8_group", "mxfp4", "qk"]
    nbytes = {"fp8_token": row_bytes("fp8_token", M, H), "fp8_group": row_bytes("fp8_group", M, H),
              "mxfp4": row_bytes("mxfp4", M, H), "qk": qk_bytes(qw.T, qw.Hq, qw.Hk, qw.D)}

    def call(name, n):
        """The n-th call of a kernel: rows rotate over the input sets, QK over its own pool."""
        s = n % args.sets
        i, o = sets[s], outs[s]
        if name == "fp8_token":
            q, ro, sc = o["t"]
            r = rq.rmsnorm_quant_fp8_per_token(i["x"], i["residual"], i["weight"], wl.eps, q_out=q, residual_out=ro,
                                               scale_out=sc)
        elif name == "fp8_group":
            q, ro, sc = o["g"]
            r = rq.rmsnorm_quant_fp8_per_group(i["x"], i["residual"], i["weight"], wl.eps, 128, q_out=q,
                                               residual_out=ro, scale_out=sc)
        elif name == "mxfp4":
            q, ro, sc = o["m"]
            r = rq.rmsnorm_quant_mxfp4(i["x"], i["residual"], i["weight"], wl.eps, q_out=q, residual_out=ro,
                                       scale_out=sc)
        else:
            r = rq.qk_gemma_rmsnorm_gate(qk_sets["qg"][n % QK_SETS], qk_sets["k"][n % QK_SETS], qd["q_w"], qd["k_w"],
                                         qw.Hq, qw.Hk, qw.D, qw.eps, q_out=qk_out[0], k_out=qk_out[1],
                                         gate_out=qk_out[2])
        if r is None:
            raise RuntimeError(f"{name}: the library refused a supported shape")

    # ---- warmup ----
    j = 0
    for w in range(args.warmup):
        for name in kernels:
            call(name, j)
            j += 1
    torch.cuda.synchronize()

    # ---- timed region: exactly K steps of work, run kernel-major ----
    # All calls are independent, so the K steps are issued as four phases of
    # K back-to-back calls (one phase per kernel, inputs rotating per call).
    # Each phase is one HIP graph, captured and uploaded before the timed
    # region (capture executes nothing), so launches go out back to back as
    # the pages time their kernels.  A HIP event at every phase boundary on the
    # launch stream gives each kernel's average launch duration as its phase
    # time / K.
    graphs = {}
    for name in kernels:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for k in range(args.steps):
                call(name, j + k)
        graphs[name] = g
    j += args.steps
    upload_graphs(torch, graphs.values(), stream)
    # Untimed replays of the step's graphs, in step order, before the timed one.
    # After the host has spent its time capturing and uploading, the first
    # replays run slower: on MI355X the timed step measured 5639-5736 GB/s
    # after one untimed replay, 5841-5862 after two, 5926-5946 after four or
    # eight, and with four its kernels run as fast as each alone.
    for _ in range(GRAPH_WARMUP_REPLAYS):
        for name in kernels:
            graphs[name].replay()
    torch.cuda.synchronize()
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(len(kernels) + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    marks[0].record(stream)
    for n, name in enumerate(kernels):
        graphs[name].replay()
        marks[n + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total_ms = marks[0].elapsed_time(marks[-1])
    ms_per_step = total_ms / args.steps
    per_kernel_us = {name: 1000.0 * marks[n].elapsed_time(marks[n + 1]) / args.steps
                     for n, name in enumerate(kernels)}
    step_bytes = sum(nbytes.values())
    value = step_bytes / (ms_per_step * 1e-3) / 1e9

    if args.profile_pass:
        # The column-major-scale calls, 4 each at ld = M then at ld = M + 64, in
        # the order fp8_group, mxfp4, so that counter runs can name each launch.
        for ld in (M, M + 64):
            gs = torch.empty((H // 128, ld), dtype=torch.float32, device=dev)
            ms = torch.empty((H // 32, ld), dtype=torch.uint8, device=dev)
            for fmt in ("fp8_group", "mxfp4"):
                for k in range(4):
                    st, o = sets[k % args.sets], outs[k % args.sets]
                    fn = rq.rmsnorm_quant_fp8_per_group_tscale if fmt == "fp8_group" else rq.rmsnorm_quant_mxfp4_tscale
                    extra = (128,) if fmt == "fp8_group" else ()
                    q, ro, _ = o["g" if fmt == "fp8_group" else "m"]
                    fn(st["x"], st["residual"], st["weight"], wl.eps, *extra, q_out=q, residual_out=ro,
                       scale_out=gs if fmt == "fp8_group" else ms)
            torch.cuda.synchronize()
        # A plain device copy of known size, for scaling the HBM byte counters.
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()

    kernels_out = {}
    for name in kernels:
        us = per_kernel_us[name]
        gbs = nbytes[name] / (us * 1e-6) / 1e9
        kernels_out[name] = {"us": round(us, 3), "bytes": nbytes[name], "GBps": round(gbs, 1),
                             "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4)}

    # Each prefill kernel alone: its own K-call graph replayed after an untimed
    # replay, the kernels taken in turn, median over the replays.  Inside the
    # step a kernel's time depends on which phase ran before it; alone it does
    # not, so the roofline kernel and its figure come from these times.
    prefill = ("fp8_token", "fp8_group", "mxfp4")
    alone = alone_us(torch, {n: graphs[n] for n in prefill}, args.steps, stream)
    alone_out = {}
    for name in prefill:
        gbs = nbytes[name] / (alone[name] * 1e-6) / 1e9
        alone_out[name] = {"us": round(alone[name], 3), "GBps": round(gbs, 1), "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4)}
    dom = max(prefill, key=lambda n: alone[n])  # the largest share of the step
    roofline = {"bound": "hbm", "kernel": f"rmsnorm_quant_{dom} [{M}, {H}]",
                "achieved": alone_out[dom]["GBps"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": alone_out[dom]["frac_of_peak"], "traffic": measured_traffic(dom),
                "timing": f"median of {ALONE_REPLAYS} replays of a {args.steps}-call graph of this kernel alone "
                          f"(HIP events on its stream)", "in_step_us": round(per_kernel_us[dom], 3)}

    result = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"prefill rows [{M}, {H}] bf16 (per-token FP8, per-group-128 FP8, MXFP4) + "
                               f"QK GemmaRMSNorm+gate T={qw.T} Hq={qw.Hq} Hk={qw.Hk} D={qw.D}",
                   "M": M, "H": H, "eps": wl.eps, "rotating_input_sets": args.sets, "step_bytes": step_bytes,
                   "graph_warmup_steps": GRAPH_WARMUP_REPLAYS * args.steps},
        "frac_of_peak": round(value / HBM_PEAK_GBS, 4),
        "kernels": kernels_out,
        "kernels_alone": alone_out,
        "roofline": roofline,
        "wall_s_timed": round(wall, 4),
    }
    if not args.no_decode and not args.profile_pass:
        result["prefill_4096x4096"] = half_batch(torch, rq, dev, sets, outs, args, stream)
        result["decode"] = decode_latency(torch, rq, inputs, dev)
        result["unfused_vs_fused"] = unfused_comparison(torch, rq, inputs, dev, sets, outs, per_kernel_us, args)
        result["qk_prefill"] = qk_prefill(torch, rq, dev)
        result["column_major_scales_8192x4096"] = transposed_scales(torch, rq, dev, sets, outs, args)
        result["fp16_rows_8192x4096"] = fp16_rows(torch, rq, dev, sets, outs, args)
    if not args.no_cpu_baseline and not args.profile_pass:
        result["cpu_baseline"] = cpu_baseline(inputs, wl, qw, nbytes)
    print(json.dumps(result), flush=True)


ALONE_REPLAYS = 7
QK_SETS = 256
GRAPH_WARMUP_REPLAYS = 4


def alone_us(torch, graphs, calls, stream, replays=ALONE_REPLAYS):
    """Median µs per call of each graph of `calls` back-to-back calls: one
    untimed replay each, then `replays` rounds replaying the graphs in turn,
    HIP events on the launch stream around each replay."""
    import statistics
    for g in graphs.values():
        g.replay()
    torch.cuda.synchronize()
    times = {n: [] for n in graphs}
    for _ in range(replays):
        for n, g in graphs.items():
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            g.replay()
            b.record(stream)
            torch.cuda.synchronize()
            times[n].append(1000.0 * a.elapsed_time(b) / calls)
    return {n: statistics.median(t) for n, t in times.items()}


def half_batch(torch, rq, dev, sets, outs, args, stream):
    """The three fused formats at [M/2, H] (4096 rows at the benchmark's shape),
    the low end of the prefill range: 2 x sets rotating input sets (each half of
    each [M, H] set, 512 MiB of inputs in all) and outputs, timed like
    alone_us."""
    M, H = sets[0]["x"].shape
    h = M // 2
    halves = [(st, o, lo) for st, o in zip(sets, outs) for lo in (0, h)]
    n = len(halves)
    key = {"fp8_token": "t", "fp8_group": "g", "mxfp4": "m"}

    def fn(fmt, k):
        st, o, lo = halves[k % n]
        q, ro, sc = o[key[fmt]]
        x, r, w = st["x"][lo:lo + h], st["residual"][lo:lo + h], st["weight"]
        if fmt == "fp8_token":
            return rq.rmsnorm_quant_fp8_per_token(x, r, w, 1e-6, q_out=q[lo:lo + h], residual_out=ro[lo:lo + h],
                                                  scale_out=sc[lo:lo + h])
        if fmt == "fp8_group":
            return rq.rmsnorm_quant_fp8_per_group(x, r, w, 1e-6, 128, q_out=q[lo:lo + h], residual_out=ro[lo:lo + h],
                                                  scale_out=sc[lo:lo + h])
        return rq.rmsnorm_quant_mxfp4(x, r, w, 1e-6, q_out=q[lo:lo + h], residual_out=ro[lo:lo + h],
                                      scale_out=sc[lo:lo + h])

    calls = 2 * args.steps
    graphs = {}
    for fmt in key:
        for k in range(n):
            fn(fmt, k)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for k in range(calls):
                fn(fmt, k)
        graphs[fmt] = g
    upload_graphs(torch, graphs.values(), stream)
    us = alone_us(torch, graphs, calls, stream)
    res = {"M": h, "H": H, "rotating_input_sets": n}
    for fmt in key:
        nb = row_bytes(fmt, h, H)
        gbs = nb / (us[fmt] * 1e-6) / 1e9
        res[fmt] = {"us": round(us[fmt], 3), "bytes": nb, "GBps": round(gbs, 1), "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4)}
    return res


def upload_graphs(torch, graphs, stream) -> None:
    """hipGraphUpload each instantiated graph, so that its first replay (the
    timed one) does not also copy the graph's launch packets to the device."""
    import ctypes
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipGraphUpload.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    hip.hipGraphUpload.restype = ctypes.c_int
    for g in graphs:
        err = hip.hipGraphUpload(ctypes.c_void_p(g.raw_cuda_graph_exec()), ctypes.c_void_p(stream.cuda_stream))
        if err != 0:
            raise RuntimeError(f"hipGraphUpload failed with error {err}")
    torch.cuda.synchronize()


def measured_traffic(kernel: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None when the kernel source changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "hbm_traffic_prefill_8192x4096.md")
    src = os.path.join(ROOT, "rmsnorm_activation_quantization_amd", "csrc", "rmsnorm_quant.hip")
    if not os.path.exists(path):
        return None
    digest = hashlib.sha256(open(src, "rb").read()).hexdigest()[:16]
    for line in open(path):
        if line.startswith("traffic-json:"):
            rec = json.loads(line.split(":", 1)[1])
            if rec.get("source_sha256_16") == digest and kernel in rec.get("bytes_per_launch", {}):
                return rec["bytes_per_launch"][kernel]
    return None


def eager_host_us(torch, rq, inputs, dev, n: int = 2000, reps: int = 5):
    """Wall time per eager call (no graph) through the Python binding at [16, 4096], the outputs
    given: median over `reps` loops of `n` calls.  The GPU keeps up (each call's kernel is shorter than
    its host time), so this is the host cost an eager decode caller pays."""
    import statistics
    wl = inputs.DECODE_4096
    d = inputs.row_inputs(wl)
    x, r, w = (d[k].to(dev) for k in ("x", "residual", "weight"))
    M, H = wl.M, wl.H
    ro = torch.empty((M, H), dtype=torch.bfloat16, device=dev)
    q8 = torch.empty((M, H), dtype=torch.float8_e4m3fn, device=dev)
    q4 = torch.empty((M, H // 2), dtype=torch.uint8, device=dev)
    st = torch.empty((M, 1), dtype=torch.float32, device=dev)
    sm = torch.empty((M, H // 32), dtype=torch.uint8, device=dev)
    calls = {"fp8_token": lambda: rq.rmsnorm_quant_fp8_per_token(x, r, w, wl.eps, residual_out=ro, q_out=q8,
                                                                 scale_out=st),
             "mxfp4": lambda: rq.rmsnorm_quant_mxfp4(x, r, w, wl.eps, residual_out=ro, q_out=q4, scale_out=sm)}
    res = {}
    for name, fn in calls.items():
        for _ in range(100):
            fn()
        torch.cuda.synchronize()
        times = []
        for _ in range(reps):
            t0 = time.perf_counter()
            for _ in range(n):
                fn()
            times.append((time.perf_counter() - t0) / n * 1e6)
            torch.cuda.synchronize()
        res[f"{name}_{M}x{H}"] = round(statistics.median(times), 2)
    return res


def decode_latency(torch, rq, inputs, dev, calls: int = 200, replays: int = 7):
    """Per-call microseconds at decode sizes: a graph of `calls` back-to-back
    calls over rotating inputs (more bytes than the Infinity Cache), replayed;
    the median replay divided by `calls`.  The launch floor is a one-element
    fill kernel timed the same way."""
    import statistics
    res = {}
    # [16, 4096] in every format (the per-group case is the outlier workload of that shape), then the
    # remaining decode workloads
    cases = [("fp8_token", inputs.DECODE_4096), ("fp8_group", inputs.FP8_GROUP_DECODE), ("mxfp4", inputs.DECODE_4096),
             ("fp8_token", inputs.FP8_TOKEN_SMALL), ("mxfp4", inputs.MXFP4_DECODE)]
    nsets = 1024  # decode sets of 256 KiB to 450 KiB: 256 MiB or more of rows in rotation

    def graph_us(fn):
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            for i in range(3):
                fn(i)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(calls):
                fn(i)
        times = []
        for _ in range(replays):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            g.replay()
            b.record()
            torch.cuda.synchronize()
            times.append(1000.0 * a.elapsed_time(b) / calls)
        return statistics.median(times)

    one = torch.zeros(1, device=dev)
    res["launch_floor_us"] = round(graph_us(lambda i: one.fill_(float(i))), 3)
    for fmt, wl in cases:
        M, H = wl.M, wl.H
        base = inputs.row_inputs(wl)
        # distinct rotating copies: a pool of distinct rows, sliced per set
        x = torch.randn(nsets, M, H, device=dev).to(torch.bfloat16)
        r = torch.randn(nsets, M, H, device=dev).to(torch.bfloat16)
        x[0].copy_(base["x"])
        r[0].copy_(base["residual"])
        w = base["weight"].to(dev)
        ro = torch.empty((M, H), dtype=torch.bfloat16, device=dev)
        if fmt == "mxfp4":
            q = torch.empty((M, H // 2), dtype=torch.uint8, device=dev)
            sc = torch.empty((M, H // 32), dtype=torch.uint8, device=dev)
            fn = lambda i: rq.rmsnorm_quant_mxfp4(x[i % nsets], r[i % nsets], w, wl.eps, q_out=q, residual_out=ro,
                                                  scale_out=sc)
        elif fmt == "fp8_group":
            q = torch.empty((M, H), dtype=torch.uint8, device=dev)
            sc = torch.empty((M, H // 128), dtype=torch.float32, device=dev)
            fn = lambda i: rq.rmsnorm_quant_fp8_per_group(x[i % nsets], r[i % nsets], w, wl.eps, 128, q_out=q,
                                                          residual_out=ro, scale_out=sc)
        else:
            q = torch.empty((M, H), dtype=torch.uint8, device=dev)
            sc = torch.empty((M,), dtype=torch.float32, device=dev)
            fn = lambda i: rq.rmsnorm_quant_fp8_per_token(x[i % nsets], r[i % nsets], w, wl.eps, q_out=q,
                                                          residual_out=ro, scale_out=sc)
        us = graph_us(fn)
        res[f"{fmt}_{M}x{H}_us"] = round(us, 3)
        del x, r
    qw = inputs.QK_DECODE
    qd = {k: v.to(dev) for k, v in inputs.qk_inputs(qw).items()}
    nq = 256
    qg = qd["qg"].unsqueeze(0).repeat(nq, 1, 1)
    kk = qd["k"].unsqueeze(0).repeat(nq, 1, 1)
    outs = [torch.empty((qw.T, h, qw.D), dtype=torch.bfloat16, device=dev) for h in (qw.Hq, qw.Hk, qw.Hq)]
    res[f"qk_{qw.T}x{qw.Hq}x{qw.Hk}x{qw.D}_us"] = round(graph_us(
        lambda i: rq.qk_gemma_rmsnorm_gate(qg[i % nq], kk[i % nq], qd["q_w"], qd["k_w"], qw.Hq, qw.Hk, qw.D, qw.eps,
                                           q_out=outs[0], k_out=outs[1], gate_out=outs[2])), 3)
    o8 = (torch.empty((qw.T, qw.Hq, qw.D), dtype=torch.uint8, device=dev),
          torch.empty((qw.T, qw.Hq), dtype=torch.float32, device=dev),
          torch.empty((qw.T, qw.Hk, qw.D), dtype=torch.uint8, device=dev),
          torch.empty((qw.T, qw.Hk), dtype=torch.float32, device=dev))
    o4 = (torch.empty((qw.T, qw.Hq, qw.D // 2), dtype=torch.uint8, device=dev),
          torch.empty((qw.T, qw.Hq, qw.D // 32), dtype=torch.uint8, device=dev),
          torch.empty((qw.T, qw.Hk, qw.D // 2), dtype=torch.uint8, device=dev),
          torch.empty((qw.T, qw.Hk, qw.D // 32), dtype=torch.uint8, device=dev))
    res[f"qk_mxfp4_{qw.T}x{qw.Hq}x{qw.Hk}x{qw.D}_us"] = round(graph_us(
        lambda i: rq.qk_gemma_rmsnorm_gate_mxfp4(qg[i % nq], kk[i % nq], qd["q_w"], qd["k_w"], qw.Hq, qw.Hk, qw.D,
                                                 qw.eps, q_out=o4[0], q_scale_out=o4[1], k_out=o4[2],
                                                 k_scale_out=o4[3], gate_out=outs[2])), 3)
    res[f"qk_fp8_{qw.T}x{qw.Hq}x{qw.Hk}x{qw.D}_us"] = round(graph_us(
        lambda i: rq.qk_gemma_rmsnorm_gate_fp8(qg[i % nq], kk[i % nq], qd["q_w"], qd["k_w"], qw.Hq, qw.Hk, qw.D,
                                               qw.eps, q_out=o8[0], q_scale_out=o8[1], k_out=o8[2],
                                               k_scale_out=o8[3], gate_out=outs[2])), 3)
    res["eager_host_us"] = eager_host_us(torch, rq, inputs, dev)
    # The pages' own MI355X figures, as context (other kernels, other machines' runs): the fused QK
    # norm + gate kernel per attention layer, the gfx950 launch floor, and the related FlyDSL hc_mix
    # gate at M = 1, 2, 4, 8, 16 (its Speed Tests table).
    res["pages_context_us"] = {"qk_gemma_rmsnorm_gate_kernel_mi355x_tp2": 4.6, "launch_floor_gfx950": 4.2,
                               "hc_mix_gate_mi355x_M1_2_4_8_16": [18.1, 18.8, 20.3, 22.1, 26.3]}
    return res


def qk_fp8_bytes(T: int, Hq: int, Hk: int, D: int) -> int:
    """qg, k and both weights read; FP8 q and k, their per-head fp32 scales and
    the bf16 gate written."""
    return 2 * (T * 2 * Hq * D + T * Hk * D + 2 * D) + T * (Hq + Hk) * D + 4 * T * (Hq + Hk) + 2 * T * Hq * D


def qk_mxfp4_bytes(T: int, Hq: int, Hk: int, D: int) -> int:
    """qg, k and both weights read; packed E2M1 q and k, their E8M0 bytes and the
    bf16 gate written."""
    return 2 * (T * 2 * Hq * D + T * Hk * D + 2 * D) + T * (Hq + Hk) * (D // 2 + D // 32) + 2 * T * Hq * D


def qk_prefill(torch, rq, dev, T: int = 8192, Hq: int = 16, Hk: int = 2, D: int = 256, calls: int = 24):
    """Both QK entry points at a prefill batch (T tokens), GB/s of algorithmic
    bytes: a graph of `calls` back-to-back calls over 3 rotating sets of inputs
    and outputs (800 MiB, more than the Infinity Cache), one uploaded replay
    timed."""
    nsets = 3
    gen = torch.Generator(device="cpu").manual_seed(1007)
    qg = [torch.randn((T, 2 * Hq * D), generator=gen).to(torch.bfloat16).to(dev) for _ in range(nsets)]
    kk = [torch.randn((T, Hk * D), generator=gen).to(torch.bfloat16).to(dev) for _ in range(nsets)]
    qw = (0.1 * torch.randn(D, generator=gen)).to(torch.bfloat16).to(dev)
    kw = (0.1 * torch.randn(D, generator=gen)).to(torch.bfloat16).to(dev)
    # outputs rotate with the inputs, so that no call's writes stay in the cache
    bf = [[torch.empty((T, h, D), dtype=torch.bfloat16, device=dev) for h in (Hq, Hk, Hq)] for _ in range(nsets)]
    f8 = [(torch.empty((T, Hq, D), dtype=torch.uint8, device=dev), torch.empty((T, Hq), dtype=torch.float32, device=dev),
           torch.empty((T, Hk, D), dtype=torch.uint8, device=dev), torch.empty((T, Hk), dtype=torch.float32, device=dev))
          for _ in range(nsets)]
    f4 = [(torch.empty((T, Hq, D // 2), dtype=torch.uint8, device=dev),
           torch.empty((T, Hq, D // 32), dtype=torch.uint8, device=dev),
           torch.empty((T, Hk, D // 2), dtype=torch.uint8, device=dev),
           torch.empty((T, Hk, D // 32), dtype=torch.uint8, device=dev)) for _ in range(nsets)]
    fns = {
        "qk_bf16": (lambda i: rq.qk_gemma_rmsnorm_gate(qg[i % nsets], kk[i % nsets], qw, kw, Hq, Hk, D, 1e-6,
                                                       q_out=bf[i % nsets][0], k_out=bf[i % nsets][1],
                                                       gate_out=bf[i % nsets][2]),
                    qk_bytes(T, Hq, Hk, D)),
        "qk_fp8": (lambda i: rq.qk_gemma_rmsnorm_gate_fp8(qg[i % nsets], kk[i % nsets], qw, kw, Hq, Hk, D, 1e-6,
                                                          q_out=f8[i % nsets][0], q_scale_out=f8[i % nsets][1],
                                                          k_out=f8[i % nsets][2], k_scale_out=f8[i % nsets][3],
                                                          gate_out=bf[i % nsets][2]),
                   qk_fp8_bytes(T, Hq, Hk, D)),
        "qk_mxfp4": (lambda i: rq.qk_gemma_rmsnorm_gate_mxfp4(qg[i % nsets], kk[i % nsets], qw, kw, Hq, Hk, D, 1e-6,
                                                              q_out=f4[i % nsets][0], q_scale_out=f4[i % nsets][1],
                                                              k_out=f4[i % nsets][2], k_scale_out=f4[i % nsets][3],
                                                              gate_out=bf[i % nsets][2]),
                     qk_mxfp4_bytes(T, Hq, Hk, D)),
    }
    res = {"T": T, "Hq": Hq, "Hk": Hk, "D": D}
    for name, (fn, nbytes) in fns.items():
        for i in range(nsets):
            fn(i)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(calls):
                fn(i)
        upload_graphs(torch, [g], torch.cuda.current_stream())
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        g.replay()
        b.record()
        torch.cuda.synchronize()
        us = 1000.0 * a.elapsed_time(b) / calls
        gbs = nbytes / (us * 1e-6) / 1e9
        res[name] = {"us": round(us, 3), "bytes": nbytes, "GBps": round(gbs, 1),
                     "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4)}
    return res


def paired_us(torch, pair, n, steps, replays: int = 5):
    """Median µs per call of two call sequences timed alternately: each is an
    uploaded graph of `steps` calls over `n` rotating sets, the two graphs
    replayed in turn `replays` times."""
    import statistics
    graphs = []
    for fn in pair:
        for j in range(n):
            fn(j)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for j in range(steps):
                fn(j)
        graphs.append(g)
    upload_graphs(torch, graphs, torch.cuda.current_stream())
    times = ([], [])
    for _ in range(replays):
        for g, t in zip(graphs, times):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            g.replay()
            b.record()
            torch.cuda.synchronize()
            t.append(1000.0 * a.elapsed_time(b) / steps)
    return statistics.median(times[0]), statistics.median(times[1])


def transposed_scales(torch, rq, dev, sets, outs, args):
    """The column-major-scale entry points at [8192, 4096] (leading dimension
    M) next to the row-major calls, timed alternately (paired_us); codes and
    residual_out reuse the rotating output sets."""
    M, H = sets[0]["x"].shape
    n = len(sets)
    g_scales = [torch.empty((H // 128, M), dtype=torch.float32, device=dev) for _ in range(n)]
    m_scales = [torch.empty((H // 32, M), dtype=torch.uint8, device=dev) for _ in range(n)]

    def args_of(j, key):
        return dict(q_out=outs[j % n][key][0], residual_out=outs[j % n][key][1])

    def xrw(j):
        return sets[j % n]["x"], sets[j % n]["residual"], sets[j % n]["weight"], 1e-6

    fns = {
        "fp8_group": (lambda j: rq.rmsnorm_quant_fp8_per_group_tscale(*xrw(j), 128, scale_out=g_scales[j % n],
                                                                      **args_of(j, "g")),
                      lambda j: rq.rmsnorm_quant_fp8_per_group(*xrw(j), 128, scale_out=outs[j % n]["g"][2],
                                                               **args_of(j, "g"))),
        "mxfp4": (lambda j: rq.rmsnorm_quant_mxfp4_tscale(*xrw(j), scale_out=m_scales[j % n], **args_of(j, "m")),
                  lambda j: rq.rmsnorm_quant_mxfp4(*xrw(j), scale_out=outs[j % n]["m"][2], **args_of(j, "m"))),
    }
    res = {}
    for fmt, pair in fns.items():
        us, row_us = paired_us(torch, pair, n, args.steps)
        nbytes = row_bytes(fmt, M, H)
        res[fmt] = {"us": round(us, 3), "GBps": round(nbytes / (us * 1e-6) / 1e9, 1),
                    "frac_of_peak": round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                    "row_major_us": round(row_us, 3)}
    return res


def fp16_rows(torch, rq, dev, sets, outs, args):
    """The fused formats on fp16 rows (the same values as the bf16 sets, cast)
    at [8192, 4096], timed alternately with the bf16 calls (paired_us); codes
    and scales reuse the rotating output sets, residual_out has fp16 buffers of
    its own."""
    M, H = sets[0]["x"].shape
    n = len(sets)
    h16 = [{k: v.to(torch.float16) for k, v in st.items()} for st in sets]
    ro16 = [torch.empty((M, H), dtype=torch.float16, device=dev) for _ in range(n)]
    calls = {"fp8_token": (rq.rmsnorm_quant_fp8_per_token, "t", ()),
             "fp8_group": (rq.rmsnorm_quant_fp8_per_group, "g", (128,)),
             "mxfp4": (rq.rmsnorm_quant_mxfp4, "m", ())}
    res = {}
    for fmt, (fn, key, extra) in calls.items():
        def f16(j, fn=fn, key=key, extra=extra):
            d = h16[j % n]
            q, _, sc = outs[j % n][key]
            return fn(d["x"], d["residual"], d["weight"], 1e-6, *extra, q_out=q, residual_out=ro16[j % n],
                      scale_out=sc)

        def bf16(j, fn=fn, key=key, extra=extra):
            d = sets[j % n]
            q, ro, sc = outs[j % n][key]
            return fn(d["x"], d["residual"], d["weight"], 1e-6, *extra, q_out=q, residual_out=ro, scale_out=sc)

        us, bf_us = paired_us(torch, (f16, bf16), n, args.steps)
        nbytes = row_bytes(fmt, M, H)
        res[fmt] = {"us": round(us, 3), "GBps": round(nbytes / (us * 1e-6) / 1e9, 1),
                    "frac_of_peak": round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4), "bf16_us": round(bf_us, 3)}
    del h16, ro16
    return res


def unfused_comparison(torch, rq, inputs, dev, sets, outs, fused_us, args):
    """The same work as the unfused sequence (rmsnorm_residual_bf16, then
    quantize_*: two launches with the bf16 row y written and read back) next
    to the fused call.  Prefill: K back-to-back pairs over the rotating sets in
    one graph, timed like the fused phases.  Decode [16, 4096]: graph replay over
    rotating cold inputs."""
    import statistics
    M, H = sets[0]["x"].shape
    ys = [torch.empty((M, H), dtype=torch.bfloat16, device=dev) for _ in sets]
    res = {"prefill_8192x4096": {}, "decode_16x4096": {}}

    def quant(fmt, y, o):
        if fmt == "fp8_token":
            return rq.quantize_fp8_per_token(y, q_out=o["t"][0], scale_out=o["t"][2])
        if fmt == "fp8_group":
            return rq.quantize_fp8_per_group(y, 128, q_out=o["g"][0], scale_out=o["g"][2])
        return rq.quantize_mxfp4(y, q_out=o["m"][0], scale_out=o["m"][2])

    key = {"fp8_token": "t", "fp8_group": "g", "mxfp4": "m"}
    for fmt in ("fp8_token", "fp8_group", "mxfp4"):
        def pair(j):
            i, o = sets[j % len(sets)], outs[j % len(sets)]
            rq.rmsnorm_residual_bf16(i["x"], i["residual"], i["weight"], 1e-6, residual_out=o[key[fmt]][1],
                                     y_out=ys[j % len(sets)])
            quant(fmt, ys[j % len(sets)], o)
        for j in range(4):
            pair(j)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for j in range(args.steps):
                pair(j)
        upload_graphs(torch, [g], torch.cuda.current_stream())
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        g.replay()
        b.record()
        torch.cuda.synchronize()
        un = 1000.0 * a.elapsed_time(b) / args.steps
        res["prefill_8192x4096"][fmt] = {"fused_us": round(fused_us[fmt], 3), "unfused_us": round(un, 3),
                                         "fused_speedup": round(un / fused_us[fmt], 3)}

    # decode
    wl = inputs.DECODE_4096
    nsets, calls = 1024, 200
    x = torch.randn(nsets, wl.M, wl.H, device=dev).to(torch.bfloat16)
    r = torch.randn(nsets, wl.M, wl.H, device=dev).to(torch.bfloat16)
    w = inputs.row_inputs(wl)["weight"].to(dev)
    o = dict(t=(torch.empty((wl.M, wl.H), dtype=torch.uint8, device=dev), None,
                torch.empty((wl.M,), dtype=torch.float32, device=dev)),
             g=(torch.empty((wl.M, wl.H), dtype=torch.uint8, device=dev), None,
                torch.empty((wl.M, wl.H // 128), dtype=torch.float32, device=dev)),
             m=(torch.empty((wl.M, wl.H // 2), dtype=torch.uint8, device=dev), None,
                torch.empty((wl.M, wl.H // 32), dtype=torch.uint8, device=dev)))
    ro = torch.empty((wl.M, wl.H), dtype=torch.bfloat16, device=dev)
    y = torch.empty((wl.M, wl.H), dtype=torch.bfloat16, device=dev)

    def graph_us(fn):
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            fn(0)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(calls):
                fn(i)
        times = []
        for _ in range(7):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            g.replay()
            b.record()
            torch.cuda.synchronize()
            times.append(1000.0 * a.elapsed_time(b) / calls)
        return statistics.median(times)

    fused_fn = {
        "fp8_token": lambda i: rq.rmsnorm_quant_fp8_per_token(x[i % nsets], r[i % nsets], w, 1e-6, residual_out=ro,
                                                              q_out=o["t"][0], scale_out=o["t"][2]),
        "fp8_group": lambda i: rq.rmsnorm_quant_fp8_per_group(x[i % nsets], r[i % nsets], w, 1e-6, 128,
                                                              residual_out=ro, q_out=o["g"][0], scale_out=o["g"][2]),
        "mxfp4": lambda i: rq.rmsnorm_quant_mxfp4(x[i % nsets], r[i % nsets], w, 1e-6, residual_out=ro,
                                                  q_out=o["m"][0], scale_out=o["m"][2]),
    }
    for fmt in ("fp8_token", "fp8_group", "mxfp4"):
        def pair(i, fmt=fmt):
            rq.rmsnorm_residual_bf16(x[i % nsets], r[i % nsets], w, 1e-6, residual_out=ro, y_out=y)
            quant(fmt, y, o)
        f = graph_us(fused_fn[fmt])
        u = graph_us(pair)
        res["decode_16x4096"][fmt] = {"fused_us": round(f, 3), "unfused_us": round(u, 3),
                                      "fused_speedup": round(u / f, 3)}
    return res


def cpu_baseline(inputs, wl, qw, nbytes):
    """The oracle as it stands (untuned, one row at a time in fp64), threaded
    over row slices (ctypes releases the GIL) on the host cores next to the GPU.
    Sample: whole steps of the benchmark's work (all rows, the three formats and
    the QK case), at least three and until about 10 s of CPU time have been
    spent; the median step.  On one thread: a slice of the rows, median of three."""
    import concurrent.futures as cf
    import statistics

    import oracle
    ref = oracle.get()
    d = inputs.row_inputs(wl)
    xb, rb, wb = (inputs.bits(d[k]) for k in ("x", "residual", "weight"))
    qd = inputs.qk_inputs(qw)
    qargs = [inputs.bits(qd[n]) for n in ("qg", "k", "q_w", "k_w")]
    # Every core of the affinity set, unless the host states a smaller thread
    # share for this process (OMP_NUM_THREADS, as a shared GPU host does).
    affinity = len(os.sched_getaffinity(0))
    share = int(os.environ.get("OMP_NUM_THREADS", "0") or 0)
    threads = max(1, min(affinity, share) if share > 0 else affinity)
    rows = wl.M
    bounds = [(i * rows // threads, (i + 1) * rows // threads) for i in range(threads)]

    def part(lo, hi):
        ref.fp8_per_token(xb[lo:hi], rb[lo:hi], wb, wl.eps)
        ref.fp8_per_group(xb[lo:hi], rb[lo:hi], wb, wl.eps, 128)
        ref.mxfp4(xb[lo:hi], rb[lo:hi], wb, wl.eps)

    step_bytes = sum(nbytes.values())
    steps = []
    cpu0 = time.process_time()
    with cf.ThreadPoolExecutor(threads) as ex:
        while len(steps) < 3 or (len(steps) < 8 and time.process_time() - cpu0 < 10.0):
            t0 = time.perf_counter()
            list(ex.map(lambda b: part(*b), bounds))
            ref.qk_gemma_rmsnorm_gate(*qargs, qw.Hq, qw.Hk, qw.D, qw.eps)
            steps.append(time.perf_counter() - t0)
    cpu_s = time.process_time() - cpu0
    # the same oracle on one thread, over one slice of the rows
    one_rows = max(1, rows // 16)
    ones = []
    for _ in range(3):
        t0 = time.perf_counter()
        part(0, one_rows)
        ones.append(time.perf_counter() - t0)
    one_bytes = sum(row_bytes(f, one_rows, wl.H) for f in ("fp8_token", "fp8_group", "mxfp4"))
    step_s, one_s = statistics.median(steps), statistics.median(ones)
    return {"value": round(step_bytes / step_s / 1e9, 3), "unit": "GB/s", "cores": threads,
            "affinity_cores": affinity, "thread_share": share or None, "kind": "oracle",
            "sample": f"{len(steps)} whole steps (the median taken): all {rows} rows of [{rows}, {wl.H}] in the "
                      f"three formats plus the QK case, threaded over row slices",
            "step_s": round(step_s, 3), "wall_s": round(sum(steps), 3), "cpu_s": round(cpu_s, 2),
            "single_thread": {"value": round(one_bytes / one_s / 1e9, 3), "unit": "GB/s", "cores": 1,
                              "sample": f"the first {one_rows} rows of [{rows}, {wl.H}] in the three formats, "
                                        f"median of 3",
                              "wall_s": round(one_s, 3)}}


if __name__ == "__main__":
    main()
