"""Seeded random configurations of the fused row entry points against the
oracle: element type, rows, row length (ragged against every tiling), format,
group size, strided inputs, in-place residual, side output, eps (including
0) and the magnitude of the rows.  Each case is printed before it runs."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import rmsnorm_activation_quantization_amd as rq
from oracle_pins import NP_CODEC
from parity import check_fp8, check_mxfp4, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
N_CASES = 48


def make_case(i: int) -> dict:
    rng = np.random.default_rng(90_000 + i)
    dtype = "fp16" if rng.random() < 0.35 else "bf16"
    fmt = ["fp8_token", "fp8_group", "mxfp4"][rng.integers(0, 3)]
    M = int(rng.choice([1, 2, 3, 7, 16, 17, 63, 64, 65, 129, 300]))
    H = int(32 * rng.integers(1, 513))                 # 32 .. 16384, multiples of 32
    if fmt == "fp8_token" and rng.random() < 0.3:
        H = int(8 * rng.integers(1, 2049))             # any multiple of 8
    group = 128
    if fmt == "fp8_group":
        choices = [g for g in (32, 64, 128, 256, 512) if H % g == 0]
        group = int(rng.choice(choices))
    return dict(dtype=dtype, fmt=fmt, M=M, H=H, group=group,
                pad_x=int(8 * rng.integers(0, 5)), pad_r=int(8 * rng.integers(0, 5)),
                inplace=bool(rng.random() < 0.25), emit_y=True,
                eps=float(0.0 if rng.random() < 0.1 else 10.0 ** rng.uniform(-8, -2)),
                mag=float(2.0 ** rng.integers(-40, 40)), seed=int(rng.integers(1 << 30)))


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_configuration(ref, i):
    c = make_case(i)
    print(f"case {i}: {c}", flush=True)
    rnd, val = NP_CODEC[c["dtype"]]
    tdt = torch.float16 if c["dtype"] == "fp16" else torch.bfloat16
    rng = np.random.default_rng(c["seed"])
    M, H = c["M"], c["H"]
    mag = c["mag"] if c["dtype"] == "bf16" else min(max(c["mag"], 2.0 ** -8), 2.0 ** 6)  # fp16: no overflow, no all-zero rows
    xb = rnd(rng.normal(0, 1, (M, H)) * mag)
    rb = rnd(rng.normal(0, 1, (M, H)) * mag)
    wb = rnd(rng.normal(1, 0.1, H))
    xw = np.zeros((M, H + c["pad_x"]), np.uint16)
    rw = np.zeros((M, H + (0 if c["inplace"] else c["pad_r"])), np.uint16)
    xw[:, :H], rw[:, :H] = xb, rb

    def dev(a):
        return torch.from_numpy(a.view(np.int16)).view(tdt).to(DEV)

    x, r, w = dev(xw)[:, :H], dev(rw)[:, :H], dev(wb)
    kw = dict(emit_y=True)
    if c["inplace"]:
        kw["residual_out"] = r
    if c["fmt"] == "fp8_token":
        out = rq.rmsnorm_quant_fp8_per_token(x, r, w, c["eps"], **kw)
    elif c["fmt"] == "fp8_group":
        out = rq.rmsnorm_quant_fp8_per_group(x, r, w, c["eps"], c["group"], **kw)
    else:
        out = rq.rmsnorm_quant_mxfp4(x, r, w, c["eps"], **kw)
    assert out is not None, "a supported configuration was refused"
    torch.cuda.synchronize()
    q, res, scale, y = out
    gpu = to_np(dict(q=q, residual_out=res, scale=scale, y=y))
    if c["fmt"] == "mxfp4":
        o = ref.mxfp4(xb, rb, wb, c["eps"], emit_y=True, dtype=c["dtype"])
        check_mxfp4(gpu, o, ref.quantize_mxfp4(gpu["y"], dtype=c["dtype"]), f"case {i}")
    else:
        g = H if c["fmt"] == "fp8_token" else c["group"]
        if c["fmt"] == "fp8_token":
            o = ref.fp8_per_token(xb, rb, wb, c["eps"], emit_y=True, dtype=c["dtype"])
        else:
            o = ref.fp8_per_group(xb, rb, wb, c["eps"], g, emit_y=True, dtype=c["dtype"])
        check_fp8(gpu, o, ref.quantize_fp8(gpu["y"], g, dtype=c["dtype"]), g, f"case {i}")


N_TSCALE_CASES = 24
TSCALE_ROWS = [1, 3, 16, 65, 300, 700, 1023, 1024, 1025, 1500, 2049, 3000, 4100, 8200]


def make_tscale_case(i: int) -> dict:
    """Column-major scales: row counts on both sides of the switch between the
    directly stored and the staged kernels (MXFP4 rows in turn), row lengths
    on every tiling (16-wave staged rows included), padded leading dimensions."""
    rng = np.random.default_rng(95_000 + i)
    dtype = "fp16" if rng.random() < 0.3 else "bf16"
    fmt = ["fp8_group", "mxfp4"][rng.integers(0, 2)]
    M = int(rng.choice(TSCALE_ROWS))
    if rng.random() < 0.4:  # the widths where the tiling switches
        H = int(rng.choice([256, 512, 1024, 2048, 4096, 5120, 7168, 7200, 8192]))
    else:
        H = int(32 * rng.integers(1, 513))
    while M * H > (1 << 24):
        H = max(32, H // 64 * 32)
    group = 32
    if fmt == "fp8_group":
        group = int(rng.choice([g for g in (32, 64, 128, 256, 512) if H % g == 0]))
    return dict(dtype=dtype, fmt=fmt, M=M, H=H, group=group, pad_ld=int(rng.integers(0, 70)),
                eps=float(0.0 if rng.random() < 0.1 else 10.0 ** rng.uniform(-8, -2)),
                seed=int(rng.integers(1 << 30)))


@pytest.mark.parametrize("i", range(N_TSCALE_CASES))
def test_random_column_major_configuration(ref, i):
    """Each column-major call must give the row-major call's codes, rows and
    scales bit for bit (transposed, padding past M untouched); small cases
    also meet the oracle bar."""
    c = make_tscale_case(i)
    print(f"tscale case {i}: {c}", flush=True)
    rnd, _ = NP_CODEC[c["dtype"]]
    tdt = torch.float16 if c["dtype"] == "fp16" else torch.bfloat16
    rng = np.random.default_rng(c["seed"])
    M, H, fmt = c["M"], c["H"], c["fmt"]
    xb, rb, wb = rnd(rng.normal(0, 1, (M, H))), rnd(rng.normal(0, 1, (M, H))), rnd(rng.normal(1, 0.1, H))

    def dev(a):
        return torch.from_numpy(a.view(np.int16)).view(tdt).to(DEV)

    x, r, w = dev(xb), dev(rb), dev(wb)
    G = H // (32 if fmt == "mxfp4" else c["group"])
    ld = M + c["pad_ld"]
    if fmt == "mxfp4":
        buf = torch.full((G, ld), 0xAB, dtype=torch.uint8, device=DEV)
        col = rq.rmsnorm_quant_mxfp4_tscale(x, r, w, c["eps"], scale_out=buf[:, :M], emit_y=True)
        row = rq.rmsnorm_quant_mxfp4(x, r, w, c["eps"], emit_y=True)
    else:
        buf = torch.full((G, ld), -7.0, dtype=torch.float32, device=DEV)
        col = rq.rmsnorm_quant_fp8_per_group_tscale(x, r, w, c["eps"], c["group"], scale_out=buf[:, :M], emit_y=True)
        row = rq.rmsnorm_quant_fp8_per_group(x, r, w, c["eps"], c["group"], emit_y=True)
    assert col is not None and row is not None, "a supported configuration was refused"
    torch.cuda.synchronize()
    q, res, sc, y = col
    assert torch.equal(q.view(torch.uint8), row[0].view(torch.uint8)), "codes differ from the row-major call's"
    assert torch.equal(res, row[1]) and torch.equal(y, row[3]), "rows differ from the row-major call's"
    assert torch.equal(sc, row[2].t()), "transposed scales differ from the row-major call's"
    pad = buf[:, M:]
    assert (pad == (0xAB if fmt == "mxfp4" else -7.0)).all(), "the padding past M was written"
    if M * H <= 1 << 21:
        gpu = to_np(dict(q=q, residual_out=res, y=y))
        gpu["scale"] = sc.t().contiguous().cpu().numpy()
        if fmt == "mxfp4":
            o = ref.mxfp4(xb, rb, wb, c["eps"], emit_y=True, dtype=c["dtype"])
            check_mxfp4(gpu, o, ref.quantize_mxfp4(gpu["y"], dtype=c["dtype"]), f"tscale case {i}")
        else:
            o = ref.fp8_per_group(xb, rb, wb, c["eps"], c["group"], emit_y=True, dtype=c["dtype"])
            check_fp8(gpu, o, ref.quantize_fp8(gpu["y"], c["group"], dtype=c["dtype"]), c["group"], f"tscale case {i}")
