"""The C-ABI library on a machine without a GPU: it loads, exports every
symbol include/rmsnorm_quant.h declares, and its deterministic preflight
rejects bad arguments before touching the HIP runtime.  Pointers here are
fake, aligned integers: the preflight never dereferences them and every case
returns before any HIP call."""

import os
import re
import subprocess

import pytest

import oracle
import rmsnorm_activation_quantization_amd as rq
from rmsnorm_activation_quantization_amd import _build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared(header):
    text = open(header).read()
    return re.findall(r"^\s*(?:rq_status|const char\s*\*|int|uint8_t|uint16_t|double)\s+(\w+)\s*\(", text, re.M)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_build.LIBRARY):
        _build.build()
    return rq.lib()


def test_every_declared_symbol_is_exported(lib):
    names = _declared(os.path.join(ROOT, "include", "rmsnorm_quant.h"))
    assert set(names) >= {"rmsnorm_quant_fp8_per_token", "rmsnorm_quant_fp8_per_group", "rmsnorm_quant_mxfp4",
                          "qk_gemma_rmsnorm_gate", "rq_status_string", "rmsnorm_residual_bf16",
                          "quantize_fp8_per_token", "quantize_fp8_per_group", "quantize_mxfp4"}
    dyn = subprocess.run(["nm", "-D", "--defined-only", _build.LIBRARY], capture_output=True, text=True).stdout
    for n in names:
        assert re.search(rf"\bT {n}$", dyn, re.M), f"{n} not exported"


def test_oracle_exports_its_header():
    ref = oracle.get()
    names = _declared(os.path.join(ROOT, "oracle", "rq_oracle.h"))
    assert len(names) >= 14
    for n in names:
        getattr(ref.lib, n)


def test_library_does_not_link_the_oracle():
    deps = subprocess.run(["ldd", _build.LIBRARY], capture_output=True, text=True).stdout
    assert "rq_oracle" not in deps
    assert "torch" not in deps


def test_status_strings(lib):
    for code in (rq.RQ_OK, rq.RQ_ERR_INVALID, rq.RQ_ERR_UNSUPPORTED, rq.RQ_ERR_HIP, rq.RQ_ERR_DEVICE):
        assert rq.status_string(code).startswith(("RQ_OK", "RQ_ERR"))
    assert "gfx950" in rq.status_string(rq.RQ_ERR_DEVICE)
    assert rq.status_string(99) == "unknown rq_status"


A = 1 << 20  # fake, 256-byte aligned device addresses, far apart
BUF = [A * (i + 1) for i in range(8)]


def row_call(lib, fn, M=4, H=256, eps=1e-6, ldx=None, ldr=None, ptrs=None, group=128):
    x, r, w, ro, q, s, y = ptrs or BUF[:7]
    ldx = H if ldx is None else ldx
    ldr = H if ldr is None else ldr
    if fn == "rmsnorm_quant_fp8_per_group":
        return lib.rmsnorm_quant_fp8_per_group(x, ldx, r, ldr, w, M, H, eps, group, ro, q, s, y, None)
    return getattr(lib, fn)(x, ldx, r, ldr, w, M, H, eps, ro, q, s, y, None)


FNS = ["rmsnorm_quant_fp8_per_token", "rmsnorm_quant_fp8_per_group", "rmsnorm_quant_mxfp4"]


@pytest.mark.parametrize("fn", FNS)
def test_row_preflight_invalid(lib, fn):
    assert row_call(lib, fn, M=-1) == rq.RQ_ERR_INVALID
    assert row_call(lib, fn, H=0) == rq.RQ_ERR_INVALID
    assert row_call(lib, fn, eps=float("nan")) == rq.RQ_ERR_INVALID
    assert row_call(lib, fn, eps=-1.0) == rq.RQ_ERR_INVALID
    assert row_call(lib, fn, ldx=128) == rq.RQ_ERR_INVALID
    assert row_call(lib, fn, ldr=8) == rq.RQ_ERR_INVALID
    for i in range(6):  # every pointer but y_out is required
        ptrs = list(BUF[:7])
        ptrs[i] = None
        assert row_call(lib, fn, ptrs=ptrs) == rq.RQ_ERR_INVALID
    # overlapping outputs: q_out inside residual_out
    ptrs = list(BUF[:7])
    ptrs[4] = ptrs[3] + 256
    assert row_call(lib, fn, ptrs=ptrs) == rq.RQ_ERR_INVALID
    # an output overlapping an input other than the in-place residual
    ptrs = list(BUF[:7])
    ptrs[3] = ptrs[0]
    assert row_call(lib, fn, ptrs=ptrs) == rq.RQ_ERR_INVALID
    # sidecar overlapping the codes
    ptrs = list(BUF[:7])
    ptrs[6] = ptrs[4]
    assert row_call(lib, fn, ptrs=ptrs) == rq.RQ_ERR_INVALID


@pytest.mark.parametrize("fn", FNS)
def test_row_preflight_unsupported(lib, fn):
    assert row_call(lib, fn, H=12) == rq.RQ_ERR_UNSUPPORTED                 # H % 8
    assert row_call(lib, fn, H=rq.RQ_MAX_HIDDEN + 8) == rq.RQ_ERR_UNSUPPORTED
    ptrs = list(BUF[:7])
    ptrs[0] += 2                                                           # x not 16-byte aligned
    assert row_call(lib, fn, ptrs=ptrs) == rq.RQ_ERR_UNSUPPORTED
    assert row_call(lib, fn, ldx=260) == rq.RQ_ERR_UNSUPPORTED              # row starts misaligned
    if fn == "rmsnorm_quant_mxfp4":
        assert row_call(lib, fn, H=48) == rq.RQ_ERR_UNSUPPORTED             # H % 32
    if fn == "rmsnorm_quant_fp8_per_group":
        assert row_call(lib, fn, group=96) == rq.RQ_ERR_UNSUPPORTED
        assert row_call(lib, fn, group=1024) == rq.RQ_ERR_UNSUPPORTED
        assert row_call(lib, fn, H=384, group=256) == rq.RQ_ERR_UNSUPPORTED  # group does not divide H
        assert row_call(lib, fn, group=0) == rq.RQ_ERR_INVALID


@pytest.mark.parametrize("fn", FNS)
def test_row_empty_batch_is_ok_without_launch(lib, fn):
    assert row_call(lib, fn, M=0, ptrs=[None] * 7) == rq.RQ_OK


def test_qk_preflight(lib):
    f = lib.qk_gemma_rmsnorm_gate
    qg, k, qw, kw, qo, ko, go = BUF[:7]
    T, Hq, Hk, D = 64, 16, 2, 256
    assert f(qg, 2 * Hq * D, k, Hk * D, qw, kw, -1, Hq, Hk, D, 1e-6, qo, ko, go, None) == rq.RQ_ERR_INVALID
    assert f(qg, 2 * Hq * D - 8, k, Hk * D, qw, kw, T, Hq, Hk, D, 1e-6, qo, ko, go, None) == rq.RQ_ERR_INVALID
    assert f(qg, 2 * Hq * D, k, Hk * D - 8, qw, kw, T, Hq, Hk, D, 1e-6, qo, ko, go, None) == rq.RQ_ERR_INVALID
    assert f(None, 2 * Hq * D, k, Hk * D, qw, kw, T, Hq, Hk, D, 1e-6, qo, ko, go, None) == rq.RQ_ERR_INVALID
    assert f(qg, 2 * Hq * D, k, Hk * D, qw, kw, T, Hq, Hk, D, float("nan"), qo, ko, go, None) == rq.RQ_ERR_INVALID
    assert f(qg, 2 * Hq * D, k, Hk * D, qw, kw, T, Hq, Hk, D, 1e-6, qo, qo, go, None) == rq.RQ_ERR_INVALID
    assert f(qg, 2 * Hq * 12, k, Hk * 12, qw, kw, T, Hq, Hk, 12, 1e-6, qo, ko, go, None) == rq.RQ_ERR_UNSUPPORTED
    assert f(qg, 2 * Hq * 1024, k, Hk * 1024, qw, kw, T, Hq, Hk, 1024, 1e-6, qo, ko, go, None) == \
        rq.RQ_ERR_UNSUPPORTED
    assert f(qg + 2, 2 * Hq * D, k, Hk * D, qw, kw, T, Hq, Hk, D, 1e-6, qo, ko, go, None) == rq.RQ_ERR_UNSUPPORTED
    assert f(None, 2 * Hq * D, None, Hk * D, None, None, 0, Hq, Hk, D, 1e-6, None, None, None, None) == rq.RQ_OK


def test_norm_preflight(lib):
    f = lib.rmsnorm_residual_bf16
    x, r, w, ro, y = BUF[:5]
    assert f(x, 256, r, 256, w, 4, 256, 1e-6, ro, None, None) == rq.RQ_ERR_INVALID       # y_out required
    assert f(x, 256, r, 256, w, -1, 256, 1e-6, ro, y, None) == rq.RQ_ERR_INVALID
    assert f(x, 256, r, 256, w, 4, 256, 1e-6, ro, ro, None) == rq.RQ_ERR_INVALID         # outputs overlap
    assert f(x, 256, r, 256, w, 4, 12, 1e-6, ro, y, None) == rq.RQ_ERR_UNSUPPORTED
    assert f(x + 2, 256, r, 256, w, 4, 256, 1e-6, ro, y, None) == rq.RQ_ERR_UNSUPPORTED
    assert f(None, 256, None, 256, None, 0, 256, 1e-6, None, None, None) == rq.RQ_OK


@pytest.mark.parametrize("fn", ["quantize_fp8_per_token", "quantize_fp8_per_group", "quantize_mxfp4"])
def test_quant_preflight(lib, fn):
    y, q, s = BUF[:3]

    def call(y=y, ldy=256, M=4, H=256, q=q, s=s, group=128):
        if fn == "quantize_fp8_per_group":
            return lib.quantize_fp8_per_group(y, ldy, M, H, group, q, s, None)
        return getattr(lib, fn)(y, ldy, M, H, q, s, None)

    assert call(M=-1) == rq.RQ_ERR_INVALID
    assert call(ldy=128) == rq.RQ_ERR_INVALID
    assert call(y=None) == rq.RQ_ERR_INVALID
    assert call(q=None) == rq.RQ_ERR_INVALID
    assert call(s=None) == rq.RQ_ERR_INVALID
    assert call(q=y + 64) == rq.RQ_ERR_INVALID                                          # codes over the input
    assert call(H=12) == rq.RQ_ERR_UNSUPPORTED
    assert call(y=y + 2) == rq.RQ_ERR_UNSUPPORTED
    assert call(M=0, y=None, q=None, s=None) == rq.RQ_OK
    if fn == "quantize_mxfp4":
        assert call(H=48) == rq.RQ_ERR_UNSUPPORTED
    if fn == "quantize_fp8_per_group":
        assert call(group=96) == rq.RQ_ERR_UNSUPPORTED
        assert call(group=0) == rq.RQ_ERR_INVALID


@pytest.mark.parametrize("fn", ["rmsnorm_quant_fp8_per_group_tscale", "rmsnorm_quant_mxfp4_tscale"])
def test_tscale_preflight(lib, fn):
    x, r, w, ro, q, s, y = BUF[:7]
    M, H = 4, 256

    def call(ld, M=M, s=s):
        if fn == "rmsnorm_quant_fp8_per_group_tscale":
            return lib.rmsnorm_quant_fp8_per_group_tscale(x, H, r, H, w, M, H, 1e-6, 128, ro, q, s, ld, y, None)
        return lib.rmsnorm_quant_mxfp4_tscale(x, H, r, H, w, M, H, 1e-6, ro, q, s, ld, None, None)

    assert call(0) == rq.RQ_ERR_INVALID               # no leading dimension
    assert call(M - 1) == rq.RQ_ERR_INVALID           # below the row count
    assert call(8, s=None) == rq.RQ_ERR_INVALID
    # the column-major span [(G - 1) * ld + M] is what must stay clear of the other buffers:
    # scales starting 4 KiB below the codes with ld = 4096 run into them, with ld = M they do not
    assert call(4096, s=q - 4096) == rq.RQ_ERR_INVALID
    assert call(8, s=ro + 64) == rq.RQ_ERR_INVALID    # inside residual_out
    assert call(1, M=0, s=None) == rq.RQ_OK


def test_qk_fp8_preflight(lib):
    f = lib.qk_gemma_rmsnorm_gate_fp8
    qg, k, qw, kw, qc, qs, kc, ks, go = BUF[:8] + [A * 9]
    T, Hq, Hk, D = 64, 16, 2, 256
    ok = (qg, 2 * Hq * D, k, Hk * D, qw, kw, T, Hq, Hk, D, 1e-6, qc, qs, kc, ks, go, None)

    def call(**kw_):
        args = list(ok)
        names = ["qg", "ld_qg", "k", "ld_k", "qw", "kw", "T", "Hq", "Hk", "D", "eps", "qc", "qs", "kc", "ks", "go"]
        for n, v in kw_.items():
            args[names.index(n)] = v
        return f(*args)

    assert call(qs=None) == rq.RQ_ERR_INVALID
    assert call(ks=None) == rq.RQ_ERR_INVALID
    assert call(qs=qc + 16) == rq.RQ_ERR_INVALID        # scales inside the codes
    assert call(qs=qs + 2) == rq.RQ_ERR_UNSUPPORTED     # misaligned fp32 scales
    assert call(qc=qc + 4) == rq.RQ_ERR_UNSUPPORTED     # codes not 8-byte aligned
    assert call(T=-1) == rq.RQ_ERR_INVALID
    assert call(T=0, qg=None, k=None, qw=None, kw=None, qc=None, qs=None, kc=None, ks=None, go=None) == rq.RQ_OK


def test_absurd_extents_are_invalid(lib):
    """Strides or counts whose extent could not be a real buffer are refused
    before any arithmetic on them can overflow."""
    x, r, w, ro, q, s, y = BUF[:7]
    huge = 1 << 62
    assert lib.rmsnorm_quant_fp8_per_token(x, huge, r, 256, w, 4, 256, 1e-6, ro, q, s, None, None) == \
        rq.RQ_ERR_INVALID
    assert lib.rmsnorm_quant_mxfp4(x, 256, r, 1 << 40, w, 1 << 20, 256, 1e-6, ro, q, s, None, None) == \
        rq.RQ_ERR_INVALID
    assert lib.quantize_fp8_per_token(y, huge, 4, 256, q, s, None) == rq.RQ_ERR_INVALID
    assert lib.rmsnorm_quant_fp8_per_group_tscale(x, 256, r, 256, w, 4, 256, 1e-6, 128, ro, q, s, huge, None,
                                                  None) == rq.RQ_ERR_INVALID
    f = lib.qk_gemma_rmsnorm_gate
    assert f(x, huge, r, 512, w, w, 4, 1, 1, 256, 1e-6, ro, q, y, None) == rq.RQ_ERR_INVALID
    assert f(x, 1 << 40, r, 1 << 40, w, w, 4, 1 << 40, 1, 256, 1e-6, ro, q, y, None) == rq.RQ_ERR_UNSUPPORTED


def test_qk_mxfp4_preflight(lib):
    f = lib.qk_gemma_rmsnorm_gate_mxfp4
    qg, k, qw, kw, qc, qs, kc, ks, go = BUF[:8] + [A * 9]
    T, Hq, Hk, D = 64, 16, 2, 256
    ok = [qg, 2 * Hq * D, k, Hk * D, qw, kw, T, Hq, Hk, D, 1e-6, qc, qs, kc, ks, go, None]
    assert f(*ok[:11], qc, None, kc, ks, go, None) == rq.RQ_ERR_INVALID              # q scales missing
    assert f(*ok[:11], qc, qc + 64, kc, ks, go, None) == rq.RQ_ERR_INVALID           # scales inside the codes
    assert f(*ok[:11], qc + 2, qs, kc, ks, go, None) == rq.RQ_ERR_UNSUPPORTED        # codes not 4-byte aligned
    assert f(qg, 2 * Hq * 40, k, Hk * 40, qw, kw, T, Hq, Hk, 40, 1e-6, qc, qs, kc, ks, go, None) == \
        rq.RQ_ERR_UNSUPPORTED                                                        # D % 32
    assert f(None, 0, None, 0, None, None, 0, Hq, Hk, D, 1e-6, None, None, None, None, None, None) == rq.RQ_ERR_INVALID
    assert f(None, 2 * Hq * D, None, Hk * D, None, None, 0, Hq, Hk, D, 1e-6, None, None, None, None, None, None) == \
        rq.RQ_OK
