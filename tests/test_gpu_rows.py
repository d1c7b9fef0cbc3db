"""GPU parity of the fused residual-add + RMSNorm + quantization entry points
against the CPU oracle (calls go through the C ABI via the binding)."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import rmsnorm_activation_quantization_amd as rq
from rmsnorm_activation_quantization_amd import inputs
from oracle_pins import (fp8_probe_case, mxfp4_probe_case, np_bf16_round, np_bf16_value, BF16_VALUE,
                         every_e8m0_byte_blocks)
from parity import check_fp8, check_mxfp4, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def gpu_call(fmt, x, r, w, eps, group=128, emit_y=True, **kw):
    if fmt == "fp8_token":
        out = rq.rmsnorm_quant_fp8_per_token(x, r, w, eps, emit_y=emit_y, **kw)
    elif fmt == "fp8_group":
        out = rq.rmsnorm_quant_fp8_per_group(x, r, w, eps, group, emit_y=emit_y, **kw)
    else:
        out = rq.rmsnorm_quant_mxfp4(x, r, w, eps, emit_y=emit_y, **kw)
    assert out is not None, f"{fmt} returned 'cannot fuse' for a supported shape"
    torch.cuda.synchronize()
    q, res, scale, y = out
    return to_np(dict(q=q, residual_out=res, scale=scale, y=y))


def oracle_call(ref, fmt, xb, rb, wb, eps, group=128):
    if fmt == "fp8_token":
        o = ref.fp8_per_token(xb, rb, wb, eps, emit_y=True)
    elif fmt == "fp8_group":
        o = ref.fp8_per_group(xb, rb, wb, eps, group, emit_y=True)
    else:
        o = ref.mxfp4(xb, rb, wb, eps, emit_y=True)
    return o


def check(ref, fmt, gpu, o, group, what):
    if fmt == "mxfp4":
        return check_mxfp4(gpu, o, ref.quantize_mxfp4(gpu["y"]), what)
    H = gpu["q"].shape[1]
    granule = H if fmt == "fp8_token" else group
    return check_fp8(gpu, o, ref.quantize_fp8(gpu["y"], granule), granule, what)


def run_case(ref, fmt, d, eps, group=128, what=""):
    x, r, w = (d[k].to(DEV) for k in ("x", "residual", "weight"))
    gpu = gpu_call(fmt, x, r, w, eps, group)
    o = oracle_call(ref, fmt, inputs.bits(d["x"]), inputs.bits(d["residual"]), inputs.bits(d["weight"]), eps, group)
    stats = check(ref, fmt, gpu, o, group, what or fmt)
    # the side output changes nothing else
    plain = gpu_call(fmt, x, r, w, eps, group, emit_y=False)
    for key in ("q", "residual_out", "scale"):
        assert np.array_equal(plain[key], gpu[key]), f"{what}: {key} depends on emit_y"
    print(f"{what or fmt}: {stats}", flush=True)
    return gpu


WORKLOADS = [
    ("fp8_token", inputs.FP8_TOKEN_SMALL),
    ("fp8_group", inputs.FP8_GROUP_DECODE),
    ("mxfp4", inputs.MXFP4_DECODE),
    ("fp8_token", inputs.DECODE_4096),
    ("fp8_group", inputs.DECODE_4096),
    ("mxfp4", inputs.DECODE_4096),
    ("fp8_token", inputs.PREFILL),
    ("fp8_group", inputs.PREFILL),
    ("mxfp4", inputs.PREFILL),
]


@pytest.mark.parametrize("fmt,wl", WORKLOADS, ids=[f"{f}-{w.name}" for f, w in WORKLOADS])
def test_workload_parity(ref, fmt, wl):
    run_case(ref, fmt, inputs.row_inputs(wl), wl.eps, what=f"{fmt}-{wl.name}")


# ragged lengths, and each side of the tiling switch (one chunk a lane while rows x waves
# fit the chip's 8192 wave slots at once: M <= 4096 at H = 1024, M <= 1024 at H = 4096,
# M <= 512 at H = 7168 and 8192)
SHAPES = [(1, 32), (1, 2048), (3, 520), (15, 4096), (16, 7168), (17, 1056), (64, 4096), (1024, 4096), (1025, 4096),
          (512, 7168), (513, 7168), (65, 7168), (257, 2080), (512, 8192), (513, 8192), (70, 8192), (4096, 1024),
          (4097, 1024), (5, 8224), (9, 16384), (100, 16384), (130, 64)]


@pytest.mark.parametrize("fmt", ["fp8_token", "fp8_group", "mxfp4"])
@pytest.mark.parametrize("M,H", SHAPES)
def test_shapes(ref, fmt, M, H):
    group = 32 if H % 128 else 128
    if fmt != "fp8_token" and H % 32:
        d = inputs.random_rows(M, H, seed=1)
        x, r, w = (d[k].to(DEV) for k in ("x", "residual", "weight"))
        fn = rq.rmsnorm_quant_mxfp4 if fmt == "mxfp4" else rq.rmsnorm_quant_fp8_per_group
        args = (x, r, w, 1e-6) if fmt == "mxfp4" else (x, r, w, 1e-6, group)
        assert fn(*args) is None, "a granule that does not divide H must be refused"
        return
    run_case(ref, fmt, inputs.random_rows(M, H, seed=7 * M + H), 1e-6, group, what=f"{fmt}-{M}x{H}")


@pytest.mark.parametrize("group", [32, 64, 128, 256, 512])
@pytest.mark.parametrize("M", [5, 300])
def test_group_sizes(ref, group, M):
    run_case(ref, "fp8_group", inputs.random_rows(M, 4096, seed=group + M), 1e-6, group, what=f"group{group}-M{M}")


@pytest.mark.parametrize("fmt", ["fp8_token", "fp8_group", "mxfp4"])
def test_strided_inputs(ref, fmt):
    M, H = 40, 2048
    d = inputs.random_rows(M, H, seed=99)
    xw = torch.zeros((M, H + 64), dtype=torch.bfloat16)
    rw = torch.zeros((M, H + 128), dtype=torch.bfloat16)
    xw[:, 8:8 + H] = d["x"]
    rw[:, 64:64 + H] = d["residual"]
    xg, rg = xw.to(DEV)[:, 8:8 + H], rw.to(DEV)[:, 64:64 + H]
    assert xg.stride(0) == H + 64 and rg.stride(0) == H + 128
    gpu = gpu_call(fmt, xg, rg, d["weight"].to(DEV), 1e-6)
    o = oracle_call(ref, fmt, inputs.bits(d["x"]), inputs.bits(d["residual"]), inputs.bits(d["weight"]), 1e-6)
    check(ref, fmt, gpu, o, 128, f"strided-{fmt}")


@pytest.mark.parametrize("fmt", ["fp8_token", "mxfp4"])
def test_in_place_residual(ref, fmt):
    M, H = 70, 4096
    d = inputs.random_rows(M, H, seed=5)
    x, w = d["x"].to(DEV), d["weight"].to(DEV)
    r1, r2 = d["residual"].to(DEV), d["residual"].to(DEV)
    a = gpu_call(fmt, x, r1, w, 1e-6)
    b = gpu_call(fmt, x, r2, w, 1e-6, residual_out=r2)
    for key in ("q", "scale", "y", "residual_out"):
        assert np.array_equal(a[key], b[key]), f"in-place {key}"
    assert np.array_equal(inputs.bits(r2), a["residual_out"])


def _probe_tensors(xb, rb, wb):
    return (inputs.from_bits(xb).to(DEV), inputs.from_bits(rb).to(DEV), inputs.from_bits(wb).to(DEV))


def test_fp8_weight_probe_goldens():
    xb, rb, wb, want, scale = fp8_probe_case()
    gpu = gpu_call("fp8_token", *_probe_tensors(xb, rb, wb), 0.0)
    assert (gpu["y"][0] == wb).all(), "probe: y must equal the weight"
    assert gpu["scale"][0, 0] == scale
    assert (gpu["q"][0] == want).all(), np.nonzero(gpu["q"][0] != want)


def test_mxfp4_weight_probe_goldens():
    xb, rb, wb, packed, bytes_ = mxfp4_probe_case()
    gpu = gpu_call("mxfp4", *_probe_tensors(xb, rb, wb), 0.0)
    assert (gpu["y"][0] == wb).all()
    assert (gpu["scale"] == bytes_).all(), (gpu["scale"], bytes_)
    assert (gpu["q"] == packed).all()


def _probe_rows(values: np.ndarray, H: int, leader: float) -> np.ndarray:
    """Rows of H weights: element 0 of every granule-sized row is `leader`, the
    rest are the values to convert (zero-padded)."""
    per_row = H - 1
    n_rows = -(-len(values) // per_row)
    w = np.zeros((n_rows, H))
    w[:, 0] = leader
    flat = np.zeros(n_rows * per_row)
    flat[: len(values)] = values
    w[:, 1:] = flat.reshape(n_rows, per_row)
    return w


def test_fp8_conversion_exhaustive(ref):
    """Every bf16 value in [-448, 448] through the fused kernel with scale 1
    (x = residual = 512, eps = 0 makes y equal the weight bit for bit)."""
    vals = BF16_VALUE[:0x43E1]
    vals = np.concatenate([vals, -vals])
    H = 4096
    w = _probe_rows(vals, H, 448.0)
    xb = np_bf16_round(np.full((1, H), 512.0))
    for i in range(w.shape[0]):
        wb = np_bf16_round(w[i])
        gpu = gpu_call("fp8_token", *_probe_tensors(xb, xb.copy(), wb), 0.0)
        assert (gpu["y"][0] == wb).all()
        o = ref.fp8_per_token(xb, xb.copy(), wb, 0.0)
        assert gpu["scale"][0, 0] == 1.0 and o["scale"][0] == 1.0
        bad = np.nonzero(gpu["q"][0] != o["q"][0])[0]
        assert len(bad) == 0, f"E4M3 codes differ for {np_bf16_value(wb[bad[:8]])}"


@pytest.mark.parametrize("k", [-100, -20, 0, 5, 60, 120])
def test_mxfp4_conversion_exhaustive(ref, k):
    """Every bf16 magnitude below 8 (times 2^k) with a block maximum 7.5 * 2^k,
    so the E8M0 byte is 127 + k and every E2M1 rounding case is exercised."""
    vals = np.ldexp(BF16_VALUE[:0x4100], k)
    vals = np.concatenate([vals, -vals])
    vals = vals[(vals != 0) & (np_bf16_value(np_bf16_round(vals)) == vals)]  # exact bf16 values only
    blocks = -(-len(vals) // 31)
    w = np.zeros((blocks, 32))
    w[:, 0] = np.ldexp(7.5, k)
    flat = np.zeros(blocks * 31)
    flat[: len(vals)] = vals
    w[:, 1:] = flat.reshape(blocks, 31)
    H = 4096
    w = np.concatenate([w.reshape(-1), np.zeros((-w.size) % H)]).reshape(-1, H)
    w = np.where(w == 0, np.ldexp(1.0, k), w)  # padding blocks keep a normal amax
    xb = np_bf16_round(np.full((1, H), 512.0))
    for i in range(w.shape[0]):
        wb = np_bf16_round(w[i])
        assert (np_bf16_value(wb) == w[i]).all()
        gpu = gpu_call("mxfp4", *_probe_tensors(xb, xb.copy(), wb), 0.0)
        o = ref.mxfp4(xb, xb.copy(), wb, 0.0)
        assert (gpu["scale"] == o["scale"]).all()
        assert (gpu["q"] == o["q"]).all(), f"E2M1 codes differ in row {i} at k={k}"


def test_mxfp4_conversion_every_scale_byte(ref):
    """Every E8M0 byte a finite bf16 block can take (0-252), through the quantize
    launch: blocks led by 2^e for e from -133 (the smallest bf16 subnormal) to
    127, whose other elements run through every bf16 magnitude below 2^(e+1),
    both signs.  Every code and byte must be the oracle's bit for bit."""
    bits = every_e8m0_byte_blocks("bf16")
    out = rq.quantize_mxfp4(inputs.from_bits(bits).to(DEV))
    assert out is not None
    torch.cuda.synchronize()
    want = ref.quantize_mxfp4(bits)
    got_q, got_s = out[0].cpu().numpy(), out[1].cpu().numpy()
    assert (got_s == want["scale"]).all(), "E8M0 bytes differ"
    assert len(np.unique(got_s)) == 253, "not every byte was reached"
    bad = np.argwhere(got_q != want["q"])
    assert len(bad) == 0, f"E2M1 codes differ at {bad[:5].tolist()}"


def test_zero_sign_tiny_and_nan(ref):
    H = 1024
    rows = []
    z = np.zeros(H, np.uint16)
    z[1::2] = 0x8000
    rows.append((z, z.copy()))                                       # +0 / -0 row
    d = inputs.random_rows(4, H, seed=1)
    xb, rb = inputs.bits(d["x"]), inputs.bits(d["residual"])
    rows.append((xb[0], rb[0]))
    nan_x = xb[1].copy()
    nan_x[17] = 0x7FC0                                               # NaN in the row
    rows.append((nan_x, rb[1]))
    xs = np.stack([r[0] for r in rows])
    rs = np.stack([r[1] for r in rows])
    wt = np_bf16_round(np.random.default_rng(2).normal(0, 1e-25, H))  # tiny weights: scale < 2^-64
    w1 = inputs.bits(d["weight"])
    for wb, label in ((w1, "normal"), (wt, "tiny")):
        for fmt in ("fp8_token", "fp8_group", "mxfp4"):
            gpu = gpu_call(fmt, *_probe_tensors(xs, rs, wb), 1e-6)
            o = oracle_call(ref, fmt, xs, rs, wb, 1e-6)
            assert (gpu["residual_out"] == o["residual_out"]).all()
            # zero row: exact, signs of zero kept
            assert (gpu["y"][0] == o["y"][0]).all()
            if fmt == "mxfp4":
                assert (gpu["scale"][0] == 0).all() and (gpu["q"][0] == o["q"][0]).all()
                assert (gpu["scale"][2] == 255).any(), "NaN block must carry E8M0 255"
                req = ref.quantize_mxfp4(gpu["y"][1:2])
                assert (gpu["q"][1] == req["q"][0]).all() and (gpu["scale"][1] == req["scale"][0]).all()
            else:
                assert (gpu["scale"][0] == 0).all() and (gpu["q"][0] == o["q"][0]).all()
                assert np.isnan(gpu["scale"][2]).any(), "NaN row must give a NaN scale"
                granule = H if fmt == "fp8_token" else 128
                req = ref.quantize_fp8(gpu["y"][1:2], granule)
                assert (gpu["q"][1] == req["q"][0]).all(), f"{label} {fmt}: codes differ from quantize(y)"
                assert np.array_equal(gpu["scale"][1].reshape(-1).view(np.uint32),
                                      req["scale"][0].view(np.uint32))


def test_determinism():
    d = inputs.row_inputs(inputs.PREFILL)
    x, r, w = (d[k].to(DEV) for k in ("x", "residual", "weight"))
    for fmt in ("fp8_token", "mxfp4"):
        a = gpu_call(fmt, x, r, w, 1e-6)
        b = gpu_call(fmt, x, r, w, 1e-6)
        for key in a:
            assert np.array_equal(a[key], b[key]), f"{fmt} {key} not deterministic"


@pytest.mark.parametrize("H", [256, 544, 2048, 4096, 7168, 8192, 16384])
def test_batch_invariance(H):
    """A row gives the same bits alone in a decode batch (more waves per row,
    one chunk a lane) and inside a prefill batch (fewer waves, two chunks a
    lane): the row's sum of squares is added in one order for every tiling.
    Also rows small enough for the rescaled re-sum (eps 0, |r| ~ 2^-60)."""
    rows = 8192 if H < 4096 else 2048  # enough rows for the two-chunk tiling at every H
    for mag, eps in ((1.0, 1e-6), (2.0 ** -60, 0.0)):
        big = inputs.random_rows(rows, H, seed=H + 11, dtype=torch.bfloat16)
        x, r, w = (big[k].to(DEV) for k in ("x", "residual", "weight"))
        x, r = (x.float() * mag).to(torch.bfloat16), (r.float() * mag).to(torch.bfloat16)
        for fmt in ("fp8_token", "fp8_group", "mxfp4"):
            if fmt == "fp8_group" and H % 128:
                continue
            whole = gpu_call(fmt, x, r, w, eps)
            for m in (1, 4, 16, 64):
                part = gpu_call(fmt, x[:m].contiguous(), r[:m].contiguous(), w, eps)
                for key in part:
                    if part[key] is None:
                        continue
                    assert np.array_equal(part[key], whole[key][:m]), \
                        f"{fmt} H={H} mag={mag}: {key} of the first {m} rows depends on the batch size"


def test_unsupported_returns_none_and_writes_nothing():
    M, H = 4, rq.RQ_MAX_HIDDEN + 8
    x = torch.randn(M, H, device=DEV).to(torch.bfloat16)
    ro = torch.full((M, H), 7.0, dtype=torch.bfloat16, device=DEV)
    assert rq.rmsnorm_quant_fp8_per_token(x, x, x[0].contiguous(), residual_out=ro) is None
    torch.cuda.synchronize()
    assert (ro == 7.0).all()
    # a row start that is not 16-byte aligned
    base = torch.randn(M, 2048 + 8, device=DEV).to(torch.bfloat16)
    xs = base[:, 1:2049]
    w = torch.ones(2048, dtype=torch.bfloat16, device=DEV)
    q = torch.full((M, 2048), 5, dtype=torch.uint8, device=DEV)
    assert rq.rmsnorm_quant_mxfp4(xs, xs, w) is None
    assert rq.rmsnorm_quant_fp8_per_token(xs, xs, w, q_out=q) is None
    torch.cuda.synchronize()
    assert (q == 5).all()


def test_invalid_raises():
    M, H = 4, 256
    x = torch.randn(M, H, device=DEV).to(torch.bfloat16)
    w = torch.ones(H, dtype=torch.bfloat16, device=DEV)
    ro = torch.empty((M, H), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(ValueError):
        rq.rmsnorm_quant_fp8_per_token(x, x, w, residual_out=ro, q_out=ro.view(torch.uint8)[:, :H])
    with pytest.raises(ValueError):
        rq.rmsnorm_quant_fp8_per_token(x, x, w, eps=-1.0)


def test_empty_batch():
    x = torch.empty((0, 4096), dtype=torch.bfloat16, device=DEV)
    w = torch.ones(4096, dtype=torch.bfloat16, device=DEV)
    out = rq.rmsnorm_quant_fp8_per_token(x, x, w)
    assert out is not None and out[0].shape == (0, 4096)
    out = rq.rmsnorm_quant_mxfp4(x, x, w)
    assert out is not None and out[2].shape == (0, 128)


@pytest.mark.parametrize("exp_field", [40, 73, 100, 127, 160, 250])
def test_every_fp8_scale_significand(ref, exp_field):
    """Per-group FP8 with 32-element groups whose maxima take all 128 bf16
    significands at one exponent (the fast division-free scale path from
    exponent field 73 up, the IEEE-division path below); y equals the weight
    exactly (x = residual = 512, eps = 0), and codes and scales must equal the
    oracle's bit for bit."""
    rng = np.random.default_rng(exp_field)
    H, g = 4096, 32
    amax_bits = ((exp_field << 7) | np.arange(128)).astype(np.uint16)
    amax = np_bf16_value(amax_bits)
    w = np.empty((128, g))
    w[:, 0] = amax * np.where(rng.random(128) < 0.5, -1, 1)
    w[:, 1:] = rng.uniform(-1, 1, (128, g - 1)) * amax[:, None]
    wb = np_bf16_round(w.reshape(-1))
    over = np.abs(np_bf16_value(wb)) > np.repeat(amax, g)
    wb[over] = (wb[over] & 0x8000) | np.repeat(amax_bits, g)[over]  # keep every element within the group's amax
    xb = np_bf16_round(np.full((1, H), 512.0))
    gpu = gpu_call("fp8_group", *_probe_tensors(xb, xb.copy(), wb), 0.0, group=g)
    o = ref.fp8_per_group(xb, xb.copy(), wb, 0.0, g)
    assert (gpu["y"][0] == wb).all()
    assert np.array_equal(gpu["scale"].view(np.uint32), o["scale"].view(np.uint32)), "scales differ"
    assert (gpu["q"] == o["q"]).all(), f"codes differ in {np.count_nonzero(gpu['q'] != o['q'])} places"


@pytest.mark.parametrize("fmt", ["fp8_token", "fp8_group", "mxfp4"])
@pytest.mark.parametrize("M,H", [(4, 4096), (70, 4096), (3, 2048), (5, 512)])
def test_tiny_rows_without_eps(ref, fmt, M, H):
    """eps = 0 and rows so small that their squares underflow fp32: the
    kernel's rescaled sum must still normalize them like the oracle."""
    d = inputs.random_rows(M, H, seed=M + H)
    scale = np.array([1e-22, 1e-30, 1e-36, 3e-39])[np.arange(M) % 4]
    xb = np_bf16_round(np_bf16_value(inputs.bits(d["x"])) * scale[:, None])
    rb = np_bf16_round(np_bf16_value(inputs.bits(d["residual"])) * scale[:, None])
    wb = inputs.bits(d["weight"])
    gpu = gpu_call(fmt, *_probe_tensors(xb, rb, wb), 0.0)
    o = oracle_call(ref, fmt, xb, rb, wb, 0.0)
    check(ref, fmt, gpu, o, 128, f"tiny-{fmt}-{M}x{H}")


@pytest.mark.parametrize("fmt", ["fp8_token", "fp8_group", "mxfp4"])
def test_batch_split_over_launches(ref, fmt):
    """A batch whose grid would pass 2^31 work-items goes out as several
    launches: at H = 32 (one wave a row) a launch holds 2^25 rows, so 2^25 + 5
    rows take two.  Every row is written (sentinels in every output are gone
    and residual_out is x + residual everywhere), and rows on each side of the
    split and at both ends match the oracle."""
    H, M, split = 32, (1 << 25) + 5, 1 << 25
    gen = torch.Generator(device=DEV).manual_seed(4242)
    x = torch.randn((M, H), generator=gen, device=DEV).to(torch.bfloat16)
    r = torch.randn((M, H), generator=gen, device=DEV).to(torch.bfloat16)
    w = (1.0 + 0.1 * torch.randn(H, generator=gen, device=DEV)).to(torch.bfloat16)
    ro = torch.full((M, H), float("nan"), dtype=torch.bfloat16, device=DEV)
    y = torch.full((M, H), float("nan"), dtype=torch.bfloat16, device=DEV)
    if fmt == "mxfp4":
        q = torch.full((M, H // 2), 0x77, dtype=torch.uint8, device=DEV)
        s = torch.full((M, H // 32), 255, dtype=torch.uint8, device=DEV)
        out = rq.rmsnorm_quant_mxfp4(x, r, w, 1e-6, q_out=q, residual_out=ro, scale_out=s, y_out=y)
    elif fmt == "fp8_group":
        q = torch.full((M, H), 0x7F, dtype=torch.uint8, device=DEV)
        s = torch.full((M, 1), float("nan"), dtype=torch.float32, device=DEV)
        out = rq.rmsnorm_quant_fp8_per_group(x, r, w, 1e-6, 32, q_out=q, residual_out=ro, scale_out=s, y_out=y)
    else:
        q = torch.full((M, H), 0x7F, dtype=torch.uint8, device=DEV)
        s = torch.full((M,), float("nan"), dtype=torch.float32, device=DEV)
        out = rq.rmsnorm_quant_fp8_per_token(x, r, w, 1e-6, q_out=q, residual_out=ro, scale_out=s, y_out=y)
    assert out is not None
    torch.cuda.synchronize()
    step = 1 << 22
    for a in range(0, M, step):
        b = min(M, a + step)
        assert torch.equal(ro[a:b], (x[a:b].float() + r[a:b].float()).to(torch.bfloat16)), f"rows {a}..{b}"
        assert not torch.isnan(y[a:b]).any(), f"y not written in rows {a}..{b}"
    if fmt == "mxfp4":
        assert (s != 255).all(), "an E8M0 byte was not written"
    else:
        assert torch.isfinite(s).all() and (s > 0).all(), "a scale was not written"
        assert (q != 0x7F).all(), "an FP8 code was not written"
    picks = np.r_[0:16, split - 16:split + 5]
    idx = torch.as_tensor(picks, device=DEV)
    gpu = to_np(dict(q=q[idx], residual_out=ro[idx], scale=s.view(M, -1)[idx], y=y[idx]))
    xb, rb, wb = (inputs.bits(t.cpu()) for t in (x[idx], r[idx], w))
    o = oracle_call(ref, fmt, xb, rb, wb, 1e-6, 32)
    print(check(ref, fmt, gpu, o, 32, f"{fmt} split {M}x{H}"), flush=True)
    del x, r, ro, y, q, s
    torch.cuda.empty_cache()


def test_tensors_on_another_device_are_refused():
    """A host tensor among device tensors is refused before any launch (the
    kernels would dereference its address on the GPU)."""
    d = inputs.random_rows(4, 256, seed=3)
    x, r, w = (d[k].to(DEV) for k in ("x", "residual", "weight"))
    for fn in (rq.rmsnorm_quant_fp8_per_token, rq.rmsnorm_quant_mxfp4, rq.rmsnorm_residual_bf16):
        with pytest.raises(ValueError, match="weight is on cpu"):
            fn(x, r, w.cpu())
        with pytest.raises(ValueError, match="residual_out is on cpu"):
            fn(x, r, w, residual_out=torch.empty(4, 256, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="y_out is on cpu"):
        rq.rmsnorm_quant_fp8_per_group(x, r, w, 1e-6, 128, y_out=torch.empty(4, 256, dtype=torch.bfloat16))
    qg = torch.zeros(2, 2 * 2 * 64, dtype=torch.bfloat16, device=DEV)
    k = torch.zeros(2, 64, dtype=torch.bfloat16, device=DEV)
    qw = torch.zeros(64, dtype=torch.bfloat16, device=DEV)
    for fn in (rq.qk_gemma_rmsnorm_gate, rq.qk_gemma_rmsnorm_gate_fp8, rq.qk_gemma_rmsnorm_gate_mxfp4):
        with pytest.raises(ValueError, match="k_w is on cpu"):
            fn(qg, k, qw, qw.cpu(), 2, 1, 64)
        assert fn(qg, k, qw, qw, 2, 1, 64) is not None
    with pytest.raises(ValueError, match="gate_out is on cpu"):
        rq.qk_gemma_rmsnorm_gate(qg, k, qw, qw, 2, 1, 64, gate_out=torch.empty(2, 2, 64, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="q_scale_out is on cpu"):
        rq.qk_gemma_rmsnorm_gate_fp8(qg, k, qw, qw, 2, 1, 64, q_scale_out=torch.empty(2, 2))
    torch.cuda.synchronize()


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("fmt", ["fp8_token", "fp8_group", "mxfp4"])
def test_inf_rows(ref, fmt, dtype):
    """Inf in a row (reading c16): row 1 holds +Inf in x; in row 2 x + residual
    overflows to -Inf.  rstd is 0 there, so the Inf element's y is NaN and the
    others signed zeros: the granule holding it gets a NaN scale (E8M0 255),
    every other granule of the row scale 0 (byte 0) and signed-zero codes.
    Everything is compared with the oracle; rows 0 and 3 are ordinary."""
    tdt = torch.float16 if dtype == "fp16" else torch.bfloat16
    M, H = 4, 512
    d = inputs.random_rows(M, H, seed=91, dtype=tdt)
    xb, rb, wb = (inputs.bits(d[k]).copy() for k in ("x", "residual", "weight"))
    inf = 0x7C00 if dtype == "fp16" else 0x7F80
    big = 0x7BFF if dtype == "fp16" else 0x7F7F   # largest finite value
    xb[1, 100] = inf
    xb[2, 300], rb[2, 300] = big | 0x8000, big | 0x8000
    dev = [inputs.from_bits(a, tdt).to(DEV) for a in (xb, rb, wb)]
    gpu = gpu_call(fmt, *dev, 1e-6)
    o = oracle_call(ref, fmt, xb, rb, wb, 1e-6) if dtype == "bf16" else \
        getattr(ref, {"fp8_token": "fp8_per_token", "fp8_group": "fp8_per_group", "mxfp4": "mxfp4"}[fmt])(
            xb, rb, wb, 1e-6, *((128,) if fmt == "fp8_group" else ()), emit_y=True, dtype="fp16")
    assert (gpu["residual_out"] == o["residual_out"]).all()
    assert gpu["residual_out"][1, 100] == inf and gpu["residual_out"][2, 300] == inf | 0x8000
    ynan = lambda y: (y & 0x7FFF) > inf
    for row, col in ((1, 100), (2, 300)):
        assert ynan(gpu["y"][row, col]) and ynan(o["y"][row, col])
        rest = np.delete(np.arange(H), col)
        assert (gpu["y"][row, rest] & 0x7FFF == 0).all() and (gpu["y"][row, rest] == o["y"][row, rest]).all()
        g = {"fp8_token": H, "fp8_group": 128, "mxfp4": 32}[fmt]
        sc, osc = gpu["scale"].reshape(M, -1)[row], o["scale"].reshape(M, -1)[row]
        if fmt == "mxfp4":
            assert sc[col // g] == 255 and osc[col // g] == 255
            assert (np.delete(sc, col // g) == 0).all() and (np.delete(osc, col // g) == 0).all()
            q, oq = gpu["q"][row].reshape(-1, g // 2), o["q"][row].reshape(-1, g // 2)
        else:
            assert np.isnan(sc[col // g]) and np.isnan(osc[col // g])
            others = np.delete(np.arange(sc.size), col // g)
            assert (sc[others] == 0).all() and (osc[others] == 0).all()
            q, oq = gpu["q"][row].reshape(-1, g), o["q"][row].reshape(-1, g)
            assert ((q[col // g] & 0x7F) == 0x7F).all()
        keep = np.delete(np.arange(q.shape[0]), col // g)
        assert (q[keep] == oq[keep]).all(), "signed-zero codes of the finite granules"
    for row in (0, 3):
        assert (gpu["y"][row] == o["y"][row]).sum() >= H - 2


@pytest.mark.parametrize("fmt", ["fp8_token", "fp8_group", "mxfp4"])
@pytest.mark.parametrize("M,H,mag", [(5, 16384, 60), (3, 4096, 100), (4, 7168, 120), (70, 2048, 64), (9, 544, 70)])
def test_huge_rows(ref, fmt, M, H, mag):
    """Rows whose fp32 sum of squares overflows (|r| around 2^mag; bf16 reaches
    2^128): the kernel sums again with r scaled by 2^-80 and must match the
    oracle (fp64) to the usual bar, instead of collapsing to rstd 0."""
    d = inputs.random_rows(M, H, seed=mag + H)
    for key in ("x", "residual"):
        d[key] = (d[key].float() * 2.0 ** mag).to(torch.bfloat16)  # exact: a power of two, no overflow
    group = 32 if H % 128 else 128
    run_case(ref, fmt, d, 1e-6, group, what=f"{fmt}-huge-{M}x{H}-2^{mag}")


@pytest.mark.parametrize("fmt", ["fp8_token", "fp8_group", "mxfp4"])
def test_zero_row_without_eps(ref, fmt):
    """An all-zero row with eps = 0 has rstd = 1/0 and y = 0 * Inf: NaN, on the
    GPU as in the oracle (the NaN's sign bit may differ).  FP8: NaN scale and
    NaN codes; MXFP4: E8M0 255.  A normal row beside it is unaffected."""
    H = 256
    d = inputs.random_rows(3, H, seed=5)
    xb, rb, wb = (inputs.bits(d[k]).copy() for k in ("x", "residual", "weight"))
    xb[0], rb[0] = 0, 0
    xb[1], rb[1] = 0x8000, 0x8000          # -0 + -0 = -0
    gpu = gpu_call(fmt, *(inputs.from_bits(a).to(DEV) for a in (xb, rb, wb)), 0.0)
    o = oracle_call(ref, fmt, xb, rb, wb, 0.0)
    assert (gpu["residual_out"] == o["residual_out"]).all()
    for row in (0, 1):
        assert ((gpu["y"][row] & 0x7FFF) > 0x7F80).all() and ((o["y"][row] & 0x7FFF) > 0x7F80).all()
        if fmt == "mxfp4":
            assert (gpu["scale"][row] == 255).all() and (o["scale"][row] == 255).all()
        else:
            assert np.isnan(gpu["scale"][row]).all() and np.isnan(o["scale"][row]).all()
            assert ((gpu["q"][row] & 0x7F) == 0x7F).all() and ((o["q"][row] & 0x7F) == 0x7F).all()
    check(ref, fmt, {k: v[2:] for k, v in gpu.items()}, {k: v[2:] for k, v in o.items()}, 128, "normal row")
