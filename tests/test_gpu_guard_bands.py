"""No kernel touches memory outside its tensors.

Writes: no kernel writes outside its outputs.  Every output lives inside a larger
buffer whose guard bands (4 KiB before and after) hold a byte pattern, and so
do the padding columns between M and the leading dimension of column-major
scales; every byte of the pattern must survive the call.  The shapes reach
every tiling: one-wave rows (H <= 512, four a workgroup), multi-wave rows with
one or two chunks a lane, 16-wave rows, a ragged last workgroup, column-major
scales stored directly and staged (MXFP4 rows in turn, with a dead second
turn), the unfused launches, fp16 rows and the three QK calls.

Reads: inputs embedded in NaN-filled buffers (NaN before and after each input,
in the gap columns of strided rows, around the weights) give outputs
bit-identical to those of clean contiguous copies, so no kernel uses a value
outside its inputs' extent (a NaN read into a row's sum or maximum would show
in every output of that row)."""

from __future__ import annotations

import math

import pytest
import torch

import rmsnorm_activation_quantization_amd as rq

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
GUARD = 4096
PATTERN = 0xA5


class Guarded:
    """Output tensors carved out of one pattern-filled byte buffer each."""

    def __init__(self, device=DEV):
        self.device = device
        self.bufs = []

    def out(self, shape, dtype, ld=None):
        """A contiguous [*shape] tensor, or with `ld` a [rows, ld] tensor whose
        columns past shape[1] are padding (column-major scales)."""
        full = (shape[0], ld) if ld is not None else tuple(shape)
        nbytes = math.prod(full) * torch.empty((), dtype=dtype).element_size()
        base = torch.full((nbytes + 2 * GUARD,), PATTERN, dtype=torch.uint8, device=self.device)
        t = base[GUARD:GUARD + nbytes].view(dtype).view(full)
        self.bufs.append((base, nbytes, shape, ld, t))
        return t

    def check(self, what):
        if torch.device(self.device).type == "cuda":
            torch.cuda.synchronize()
        for base, nbytes, shape, ld, t in self.bufs:
            assert (base[:GUARD] == PATTERN).all(), f"{what}: write before an output of {tuple(t.shape)}"
            assert (base[GUARD + nbytes:] == PATTERN).all(), f"{what}: write after an output of {tuple(t.shape)}"
            if ld is not None and ld > shape[1]:
                pad = t[:, shape[1]:].contiguous().view(torch.uint8)
                assert (pad == PATTERN).all(), f"{what}: write into the padding columns of the column-major scales"


def rows(M, H, dtype=torch.bfloat16, seed=0):
    g = torch.Generator(device=DEV).manual_seed(seed + M * 131 + H)
    x = torch.randn(M, H, generator=g, device=DEV).to(dtype)
    r = torch.randn(M, H, generator=g, device=DEV).to(dtype)
    w = (1 + 0.1 * torch.randn(H, generator=g, device=DEV)).to(dtype)
    return x, r, w


SHAPES = [(1, 256), (7, 512), (3, 1024), (17, 2048), (5, 4096), (1025, 4096), (2050, 4096), (9, 5120),
          (1, 7168), (16, 7168), (1030, 7168), (3, 16384)]


@pytest.mark.parametrize("M,H", SHAPES)
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
def test_row_calls_write_only_their_outputs(M, H, dtype):
    x, r, w = rows(M, H, dtype)
    for fmt in ("fp8_token", "fp8_group", "mxfp4"):
        g = Guarded()
        ro, y = g.out((M, H), dtype), g.out((M, H), dtype)
        if fmt == "mxfp4":
            q, s = g.out((M, H // 2), torch.uint8), g.out((M, H // 32), torch.uint8)
            out = rq.rmsnorm_quant_mxfp4(x, r, w, 1e-6, q_out=q, residual_out=ro, scale_out=s, y_out=y)
        elif fmt == "fp8_group":
            q, s = g.out((M, H), torch.uint8), g.out((M, H // 128), torch.float32)
            out = rq.rmsnorm_quant_fp8_per_group(x, r, w, 1e-6, 128, q_out=q, residual_out=ro, scale_out=s, y_out=y)
        else:
            q, s = g.out((M, H), torch.uint8), g.out((M, 1), torch.float32)
            out = rq.rmsnorm_quant_fp8_per_token(x, r, w, 1e-6, q_out=q, residual_out=ro, scale_out=s, y_out=y)
        assert out is not None
        g.check(f"{fmt} [{M}, {H}] {dtype}")


@pytest.mark.parametrize("M,H", SHAPES)
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
def test_column_major_scales_write_only_their_columns(M, H, dtype):
    x, r, w = rows(M, H, dtype)
    for fmt in ("fp8_group", "mxfp4"):
        for ld in (M, M + 24):
            g = Guarded()
            ro = g.out((M, H), dtype)
            if fmt == "mxfp4":
                q = g.out((M, H // 2), torch.uint8)
                s = g.out((H // 32, M), torch.uint8, ld=ld)
                out = rq.rmsnorm_quant_mxfp4_tscale(x, r, w, 1e-6, q_out=q, residual_out=ro, scale_out=s)
            else:
                q = g.out((M, H), torch.uint8)
                s = g.out((H // 128, M), torch.float32, ld=ld)
                out = rq.rmsnorm_quant_fp8_per_group_tscale(x, r, w, 1e-6, 128, q_out=q, residual_out=ro, scale_out=s)
            assert out is not None
            g.check(f"{fmt} column-major [{M}, {H}] ld {ld} {dtype}")


@pytest.mark.parametrize("M,H", [(1, 256), (17, 2048), (1025, 4096), (16, 7168)])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
def test_unfused_launches_write_only_their_outputs(M, H, dtype):
    x, r, w = rows(M, H, dtype)
    g = Guarded()
    ro, y = g.out((M, H), dtype), g.out((M, H), dtype)
    assert rq.rmsnorm_residual_bf16(x, r, w, 1e-6, residual_out=ro, y_out=y) is not None
    q8, st, sg = g.out((M, H), torch.uint8), g.out((M, 1), torch.float32), g.out((M, H // 128), torch.float32)
    q4, sm = g.out((M, H // 2), torch.uint8), g.out((M, H // 32), torch.uint8)
    assert rq.quantize_fp8_per_token(y, q_out=q8, scale_out=st) is not None
    assert rq.quantize_fp8_per_group(y, 128, q_out=q8, scale_out=sg) is not None
    assert rq.quantize_mxfp4(y, q_out=q4, scale_out=sm) is not None
    g.check(f"unfused [{M}, {H}] {dtype}")


@pytest.mark.parametrize("T,Hq,Hk,D", [(1, 16, 2, 256), (64, 16, 2, 256), (7, 4, 1, 64), (257, 8, 8, 128),
                                       (3, 2, 2, 512)])
def test_qk_calls_write_only_their_outputs(T, Hq, Hk, D):
    gen = torch.Generator(device=DEV).manual_seed(T * 7 + D)
    qg = torch.randn(T, 2 * Hq * D, generator=gen, device=DEV).to(torch.bfloat16)
    k = torch.randn(T, Hk * D, generator=gen, device=DEV).to(torch.bfloat16)
    qw = (0.1 * torch.randn(D, generator=gen, device=DEV)).to(torch.bfloat16)
    g = Guarded()
    q, kk, gate = g.out((T, Hq, D), torch.bfloat16), g.out((T, Hk, D), torch.bfloat16), g.out((T, Hq, D), torch.bfloat16)
    assert rq.qk_gemma_rmsnorm_gate(qg, k, qw, qw, Hq, Hk, D, q_out=q, k_out=kk, gate_out=gate) is not None
    qc, qs = g.out((T, Hq, D), torch.uint8), g.out((T, Hq), torch.float32)
    kc, ks = g.out((T, Hk, D), torch.uint8), g.out((T, Hk), torch.float32)
    assert rq.qk_gemma_rmsnorm_gate_fp8(qg, k, qw, qw, Hq, Hk, D, q_out=qc, q_scale_out=qs, k_out=kc,
                                        k_scale_out=ks, gate_out=gate) is not None
    qc4, qs4 = g.out((T, Hq, D // 2), torch.uint8), g.out((T, Hq, D // 32), torch.uint8)
    kc4, ks4 = g.out((T, Hk, D // 2), torch.uint8), g.out((T, Hk, D // 32), torch.uint8)
    assert rq.qk_gemma_rmsnorm_gate_mxfp4(qg, k, qw, qw, Hq, Hk, D, q_out=qc4, q_scale_out=qs4, k_out=kc4,
                                          k_scale_out=ks4, gate_out=gate) is not None
    g.check(f"qk T={T} Hq={Hq} Hk={Hk} D={D}")


NAN_LEAD, NAN_GAP = 64, 64  # elements: 128-byte offsets keep every row start 16-byte aligned


def nan_embedded(t, device=DEV):
    """The values of `t` ([H] or [M, H]) as a view inside a NaN-filled buffer:
    NaN before and after, and (2-D) NaN in the gap columns of each row."""
    if t.dim() == 1:
        buf = torch.full((NAN_LEAD + t.numel() + NAN_LEAD,), float("nan"), dtype=t.dtype, device=device)
        v = buf[NAN_LEAD:NAN_LEAD + t.numel()]
    else:
        M, H = t.shape
        ld = H + NAN_GAP
        buf = torch.full((NAN_LEAD + M * ld + NAN_LEAD,), float("nan"), dtype=t.dtype, device=device)
        v = buf[NAN_LEAD:NAN_LEAD + M * ld].view(M, ld)[:, :H]
    v.copy_(t)
    return v


def same_bits(a, b, what):
    for i, (u, v) in enumerate(zip(a, b)):
        if u is None:
            assert v is None, what
            continue
        assert torch.equal(u.contiguous().view(torch.uint8), v.contiguous().view(torch.uint8)), f"{what}: output {i}"


@pytest.mark.parametrize("M,H", SHAPES)
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
def test_row_calls_read_only_their_inputs(M, H, dtype):
    x, r, w = rows(M, H, dtype, seed=1)
    xn, rn, wn = nan_embedded(x), nan_embedded(r), nan_embedded(w)
    calls = {
        "fp8_token": lambda *a: rq.rmsnorm_quant_fp8_per_token(*a, 1e-6, emit_y=True),
        "fp8_group": lambda *a: rq.rmsnorm_quant_fp8_per_group(*a, 1e-6, 128, emit_y=True),
        "mxfp4": lambda *a: rq.rmsnorm_quant_mxfp4(*a, 1e-6, emit_y=True),
    }
    calls["fp8_group_tscale"] = lambda *a: rq.rmsnorm_quant_fp8_per_group_tscale(*a, 1e-6, 128, emit_y=True)
    calls["mxfp4_tscale"] = lambda *a: rq.rmsnorm_quant_mxfp4_tscale(*a, 1e-6, emit_y=True)
    calls["norm"] = lambda *a: rq.rmsnorm_residual_bf16(*a, 1e-6)  # the fp16 norm launch for fp16 rows
    for name, fn in calls.items():
        same_bits(fn(x, r, w), fn(xn, rn, wn), f"{name} [{M}, {H}] {dtype}")
    y = rq.rmsnorm_residual_bf16(x, r, w, 1e-6)[1]
    yn = nan_embedded(y)
    for name in ("quantize_fp8_per_token", "quantize_mxfp4"):
        same_bits(getattr(rq, name)(y), getattr(rq, name)(yn), f"{name} [{M}, {H}] {dtype}")
    same_bits(rq.quantize_fp8_per_group(y, 128), rq.quantize_fp8_per_group(yn, 128), f"quantize group [{M}, {H}] {dtype}")
    torch.cuda.synchronize()


@pytest.mark.parametrize("T,Hq,Hk,D", [(1, 16, 2, 256), (64, 16, 2, 256), (7, 4, 1, 64), (257, 8, 8, 128),
                                       (3, 2, 2, 512)])
def test_qk_calls_read_only_their_inputs(T, Hq, Hk, D):
    gen = torch.Generator(device=DEV).manual_seed(T * 11 + D)
    qg = torch.randn(T, 2 * Hq * D, generator=gen, device=DEV).to(torch.bfloat16)
    k = torch.randn(T, Hk * D, generator=gen, device=DEV).to(torch.bfloat16)
    qw = (0.1 * torch.randn(D, generator=gen, device=DEV)).to(torch.bfloat16)
    kw = (0.1 * torch.randn(D, generator=gen, device=DEV)).to(torch.bfloat16)
    clean, embedded = (qg, k, qw, kw), tuple(nan_embedded(t) for t in (qg, k, qw, kw))
    for name in ("qk_gemma_rmsnorm_gate", "qk_gemma_rmsnorm_gate_fp8", "qk_gemma_rmsnorm_gate_mxfp4"):
        fn = getattr(rq, name)
        same_bits(fn(*clean, Hq, Hk, D), fn(*embedded, Hq, Hk, D), f"{name} T={T} Hq={Hq} Hk={Hk} D={D}")
    torch.cuda.synchronize()
