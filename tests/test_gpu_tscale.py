"""GPU parity of the column-major-scale entry points (rmsnorm_quant_fp8_per_group_tscale,
rmsnorm_quant_mxfp4_tscale and their fp16 names): against the oracle's transposed-scale
functions, and bit for bit against the row-major calls on the same rows (the same kernel
computes both; only where the scales are stored differs).  Padding columns of the scale
array past M must stay untouched."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import rmsnorm_activation_quantization_amd as rq
from rmsnorm_activation_quantization_amd import inputs
from parity import check_fp8, check_mxfp4, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
# Small batches store each column-major scale from the lane that computes it
# (every case below 1024 rows, and 3000 x 256); batches of at least 1024 rows
# whose launch fills the chip's wave slots stage the scales in LDS and store
# runs along M, MXFP4 taking two multi-wave rows in turn a workgroup
# (1100 x 4096, 8192 x 4096; 8200 x 256 with four one-wave rows a workgroup;
# the mixed-row test below adds odd counts, whose last MXFP4 workgroup has its
# second turn past the end; 1025 x 7168 and 1030 x 8192 take 16 waves with one
# chunk a lane, the staged tiling of rows that wide).  The small
# cases take every tiling of the direct stores, 520 x 7168 with two chunks a
# lane.  At H = 16384 the small cases take the direct stores' 16-wave rows and
# 1024 x 16384 fills the staged kernels' LDS stage exactly (512 E8M0 bytes;
# 512 fp32 scales at group 32).
CASES = [("bf16", 16, 4096, 128), ("bf16", 16, 7168, 32), ("bf16", 3, 544, 32), ("bf16", 130, 1024, 512),
         ("bf16", 65, 4096, 64), ("fp16", 17, 2048, 128), ("fp16", 9, 16384, 256), ("bf16", 8192, 4096, 128),
         ("bf16", 3000, 256, 32), ("bf16", 1100, 4096, 128), ("fp16", 700, 2048, 64), ("bf16", 5, 16384, 32),
         ("bf16", 520, 7168, 64), ("bf16", 8200, 256, 32), ("bf16", 1024, 16384, 32), ("bf16", 1030, 8192, 128)]


def padded(M):
    return ((M + 3) // 4) * 4 + 4  # a padded leading dimension, as blockwise GEMMs ask for


@pytest.mark.parametrize("dtype,M,H,group", CASES, ids=[f"{d}-{m}x{h}-g{g}" for d, m, h, g in CASES])
def test_tscale_fp8_group(ref, dtype, M, H, group):
    tdt = torch.float16 if dtype == "fp16" else torch.bfloat16
    d = inputs.random_rows(M, H, seed=M * 31 + H + group, dtype=tdt)
    x, r, w = (d[k].to(DEV) for k in ("x", "residual", "weight"))
    G, ld = H // group, padded(M)
    buf = torch.full((G, ld), -7.0, dtype=torch.float32, device=DEV)
    out = rq.rmsnorm_quant_fp8_per_group_tscale(x, r, w, 1e-6, group, scale_out=buf, emit_y=True)
    row = rq.rmsnorm_quant_fp8_per_group(x, r, w, 1e-6, group, emit_y=True)
    assert out is not None and row is not None
    torch.cuda.synchronize()
    q, ro, sc, y = out
    assert sc.data_ptr() == buf.data_ptr()
    assert torch.equal(q.view(torch.uint8), row[0].view(torch.uint8)) and torch.equal(ro, row[1]) and torch.equal(y, row[3])
    assert torch.equal(sc[:, :M], row[2].t()), "transposed scales differ from the row-major call's"
    assert (sc[:, M:] == -7.0).all(), "the padding past M was written"
    if M * H <= 1 << 22:
        xb, rb, wb = (inputs.bits(d[k]) for k in ("x", "residual", "weight"))
        o = ref.fp8_per_group_tscale(xb, rb, wb, 1e-6, group, ld_scale=ld, emit_y=True, dtype=dtype)
        gpu = to_np(dict(q=q, residual_out=ro, y=y))
        gpu["scale"] = sc[:, :M].t().contiguous().cpu().numpy()
        want = dict(o, scale=np.ascontiguousarray(o["scale"][:, :M].T))
        check_fp8(gpu, want, ref.quantize_fp8(gpu["y"], group, dtype=dtype), group, f"tscale {dtype} {M}x{H}")


@pytest.mark.parametrize("dtype,M,H,group", CASES, ids=[f"{d}-{m}x{h}" for d, m, h, g in CASES])
def test_tscale_mxfp4(ref, dtype, M, H, group):
    tdt = torch.float16 if dtype == "fp16" else torch.bfloat16
    d = inputs.random_rows(M, H, seed=M * 37 + H, dtype=tdt)
    x, r, w = (d[k].to(DEV) for k in ("x", "residual", "weight"))
    B, ld = H // 32, padded(M)
    buf = torch.full((B, ld), 0xAB, dtype=torch.uint8, device=DEV)
    out = rq.rmsnorm_quant_mxfp4_tscale(x, r, w, 1e-6, scale_out=buf, emit_y=True)
    row = rq.rmsnorm_quant_mxfp4(x, r, w, 1e-6, emit_y=True)
    assert out is not None and row is not None
    torch.cuda.synchronize()
    q, ro, sc, y = out
    assert torch.equal(q, row[0]) and torch.equal(ro, row[1]) and torch.equal(y, row[3])
    assert torch.equal(sc[:, :M], row[2].t()), "transposed E8M0 bytes differ from the row-major call's"
    assert (sc[:, M:] == 0xAB).all(), "the padding past M was written"
    if M * H <= 1 << 22:
        xb, rb, wb = (inputs.bits(d[k]) for k in ("x", "residual", "weight"))
        o = ref.mxfp4_tscale(xb, rb, wb, 1e-6, ld_scale=ld, emit_y=True, dtype=dtype)
        gpu = to_np(dict(q=q, residual_out=ro, y=y))
        gpu["scale"] = sc[:, :M].t().contiguous().cpu().numpy()
        want = dict(o, scale=np.ascontiguousarray(o["scale"][:, :M].T))
        check_mxfp4(gpu, want, ref.quantize_mxfp4(gpu["y"], dtype=dtype), f"tscale mx {dtype} {M}x{H}")


def test_tscale_default_and_errors():
    d = inputs.random_rows(4, 256, seed=5)
    x, r, w = (d[k].to(DEV) for k in ("x", "residual", "weight"))
    q, _, sc, _ = rq.rmsnorm_quant_fp8_per_group_tscale(x, r, w, 1e-6, 64)
    assert sc.shape == (4, 4)  # [H / group, M] by default
    with pytest.raises(ValueError):  # fewer columns than rows
        rq.rmsnorm_quant_mxfp4_tscale(x, r, w, 1e-6, scale_out=torch.empty((8, 3), dtype=torch.uint8, device=DEV))
    with pytest.raises(ValueError):  # a wrong-sized row-major output is refused before the launch
        rq.rmsnorm_quant_fp8_per_group(x, r, w, 1e-6, 64, scale_out=torch.empty((4, 3), device=DEV))
    empty = torch.empty((0, 256), dtype=torch.bfloat16, device=DEV)
    out = rq.rmsnorm_quant_mxfp4_tscale(empty, empty, w, 1e-6)
    assert out is not None and out[2].shape == (8, 1)


@pytest.mark.parametrize("M,H", [(8, 4096), (12, 1024), (6, 8192), (64, 2048)])
def test_tscale_tiny_and_normal_rows_share_a_workgroup(M, H):
    """Rows whose squares underflow (eps = 0, |r| ~ 2^-70, the rescaled sum) next
    to ordinary rows in the same workgroup (four one-wave rows at once, or two
    multi-wave MXFP4 rows in turn): the column-major calls must give the
    row-major calls' bits."""
    d = inputs.random_rows(M, H, seed=M + H, dtype=torch.bfloat16)
    x, r, w = (d[k].to(DEV) for k in ("x", "residual", "weight"))
    tiny = torch.zeros(M, 1, device=DEV)
    tiny[0::2] = 1.0
    scale = torch.where(tiny > 0, torch.tensor(2.0 ** -70, device=DEV), torch.tensor(1.0, device=DEV))
    x = (x.float() * scale).to(torch.bfloat16)
    r = (r.float() * scale).to(torch.bfloat16)
    for tfn, rfn, kw in ((rq.rmsnorm_quant_fp8_per_group_tscale, rq.rmsnorm_quant_fp8_per_group, dict(group=64)),
                         (rq.rmsnorm_quant_mxfp4_tscale, rq.rmsnorm_quant_mxfp4, {})):
        a = tfn(x, r, w, 0.0, emit_y=True, **kw)
        b = rfn(x, r, w, 0.0, emit_y=True, **kw)
        torch.cuda.synchronize()
        assert torch.equal(a[3], b[3]) and torch.equal(a[1], b[1]), "y or residual_out differs"
        assert torch.equal(a[0].view(torch.uint8), b[0].view(torch.uint8)), "codes differ"
        assert torch.equal(a[2][:, :M], b[2].t()), "scales differ"


MIXED = [(2049, 4096), (4101, 1024), (5001, 2048), (1025, 7168)]


@pytest.mark.parametrize("M,H", MIXED, ids=[f"{m}x{h}" for m, h in MIXED])
def test_tscale_mxfp4_mixed_rows_in_a_workgroup(ref, M, H):
    """MXFP4 with column-major scales takes two multi-wave rows in turn a
    workgroup at these shapes.  Rows whose fp32 sum of squares overflows
    (|r| ~ 2^70) or underflows (|r| ~ 2^-60 with eps = 0) take a second,
    rescaled sum with a barrier of its own; here they sit beside ordinary rows
    in the same workgroups (and a dead row pads the last one), one turn taking
    that barrier and the other not.  Everything must equal the row-major call
    bit for bit and meet the oracle bar."""
    d = inputs.random_rows(M, H, seed=M + H)
    idx = torch.arange(M)
    scale = torch.ones(M)
    scale[idx % 5 == 0] = 2.0 ** 70
    scale[idx % 7 == 2] = 2.0 ** -60
    for key in ("x", "residual"):
        d[key] = (d[key].float() * scale[:, None]).to(torch.bfloat16)  # exact: powers of two
    x, r, w = (d[k].to(DEV) for k in ("x", "residual", "weight"))
    ld = padded(M)
    buf = torch.full((H // 32, ld), 0xAB, dtype=torch.uint8, device=DEV)
    out = rq.rmsnorm_quant_mxfp4_tscale(x, r, w, 0.0, scale_out=buf, emit_y=True)
    row = rq.rmsnorm_quant_mxfp4(x, r, w, 0.0, emit_y=True)
    assert out is not None and row is not None
    torch.cuda.synchronize()
    q, ro, sc, y = out
    assert torch.equal(q, row[0]) and torch.equal(ro, row[1]) and torch.equal(y, row[3])
    assert torch.equal(sc[:, :M], row[2].t()), "transposed E8M0 bytes differ from the row-major call's"
    assert (sc[:, M:] == 0xAB).all(), "the padding past M was written"
    xb, rb, wb = (inputs.bits(d[k]) for k in ("x", "residual", "weight"))
    o = ref.mxfp4(xb, rb, wb, 0.0, emit_y=True)
    gpu = to_np(dict(q=q, residual_out=ro, y=y))
    gpu["scale"] = sc[:, :M].t().contiguous().cpu().numpy()
    check_mxfp4(gpu, o, ref.quantize_mxfp4(gpu["y"]), f"tscale mixed {M}x{H}")
