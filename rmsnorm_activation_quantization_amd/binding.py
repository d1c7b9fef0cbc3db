"""Thin binding of librmsnorm_quant.so (argument marshalling only).

Every entry point has the name of the C function it calls (include/rmsnorm_quant.h).
torch supplies device memory and the current stream; every step of the
computation runs in the library's HIP kernels.  Every call hands its tensors
to the marshalling module built beside this file (csrc/marshal.cpp), which
checks the arguments on torch's C++ tensors, allocates missing outputs and
calls the C entry point whose address this module resolves from the loaded
library.  There is no other code path: if the library or the marshalling
module is missing (RuntimeError at the first call) or the device is not an
MI355X (RQ_ERR_DEVICE, RuntimeError), calls fail loudly.

bf16 and fp16 rows: every row function dispatches on the dtype of x (or y):
bf16 tensors run the bf16 kernels, fp16 tensors the _f16 ones, and the row
outputs come back in the input's dtype (the activation dtype is carried
through the step).  Mixing dtypes raises ValueError.

Return convention, following sglang PR #29723 (Key changes: the fused call
returns its tuple, or None when the backend cannot fuse so that the caller runs
the unfused sequence): a tuple on success; None for RQ_ERR_UNSUPPORTED (a shape
or alignment the kernels do not take), which the library decides before
enqueuing anything; ValueError for RQ_ERR_INVALID; RuntimeError for
RQ_ERR_DEVICE and RQ_ERR_HIP.
"""

from __future__ import annotations

import ctypes
import os
import threading

import torch  # noqa: F401  (the marshalling module needs torch's Python bindings initialized)

from . import _build

RQ_OK, RQ_ERR_INVALID, RQ_ERR_UNSUPPORTED, RQ_ERR_HIP, RQ_ERR_DEVICE = 0, 1, 2, 3, 4
RQ_MAX_HIDDEN = 16384
RQ_MAX_HEAD_DIM = 512

_lib = None
_lock = threading.Lock()

_p = ctypes.c_void_p
_i64 = ctypes.c_int64
_f32 = ctypes.c_float

_SIGNATURES = {
    "rmsnorm_quant_fp8_per_token": [_p, _i64, _p, _i64, _p, _i64, _i64, _f32, _p, _p, _p, _p, _p],
    "rmsnorm_quant_fp8_per_group": [_p, _i64, _p, _i64, _p, _i64, _i64, _f32, _i64, _p, _p, _p, _p, _p],
    "rmsnorm_quant_mxfp4": [_p, _i64, _p, _i64, _p, _i64, _i64, _f32, _p, _p, _p, _p, _p],
    "rmsnorm_quant_fp8_per_group_tscale": [_p, _i64, _p, _i64, _p, _i64, _i64, _f32, _i64, _p, _p, _p, _i64, _p, _p],
    "rmsnorm_quant_mxfp4_tscale": [_p, _i64, _p, _i64, _p, _i64, _i64, _f32, _p, _p, _p, _i64, _p, _p],
    "qk_gemma_rmsnorm_gate": [_p, _i64, _p, _i64, _p, _p, _i64, _i64, _i64, _i64, _f32, _p, _p, _p, _p],
    "qk_gemma_rmsnorm_gate_fp8": [_p, _i64, _p, _i64, _p, _p, _i64, _i64, _i64, _i64, _f32, _p, _p, _p, _p, _p,
                                  _p],
    "qk_gemma_rmsnorm_gate_mxfp4": [_p, _i64, _p, _i64, _p, _p, _i64, _i64, _i64, _i64, _f32, _p, _p, _p, _p, _p,
                                    _p],
    "rmsnorm_residual_bf16": [_p, _i64, _p, _i64, _p, _i64, _i64, _f32, _p, _p, _p],
    "quantize_fp8_per_token": [_p, _i64, _i64, _i64, _p, _p, _p],
    "quantize_fp8_per_group": [_p, _i64, _i64, _i64, _i64, _p, _p, _p],
    "quantize_mxfp4": [_p, _i64, _i64, _i64, _p, _p, _p],
}
# fp16 variants of the row entry points (same arguments)
for _name in ("rmsnorm_quant_fp8_per_token", "rmsnorm_quant_fp8_per_group", "rmsnorm_quant_mxfp4",
              "rmsnorm_quant_fp8_per_group_tscale", "rmsnorm_quant_mxfp4_tscale",
              "quantize_fp8_per_token", "quantize_fp8_per_group", "quantize_mxfp4"):
    _SIGNATURES[_name + "_f16"] = _SIGNATURES[_name]
_SIGNATURES["rmsnorm_residual_f16"] = _SIGNATURES["rmsnorm_residual_bf16"]



_FN_CACHE: dict = {}


def _entries(name: str) -> tuple:
    """Addresses of the bf16 and fp16 C entry points of one row call in the
    loaded library (bf16: name, or name_bf16 for the norm launch; fp16:
    name_f16), for the marshalling module."""
    key = ("addresses", name)
    e = _FN_CACHE.get(key)
    if e is None:
        h = lib()
        bf = getattr(h, name + ("_bf16" if name == "rmsnorm_residual" else ""))
        e = (ctypes.cast(bf, ctypes.c_void_p).value, ctypes.cast(getattr(h, name + "_f16"), ctypes.c_void_p).value)
        _FN_CACHE[key] = e
    return e


def _entry(name: str) -> int:
    """Address of one C entry point of the loaded library."""
    key = ("address", name)
    e = _FN_CACHE.get(key)
    if e is None:
        e = _FN_CACHE[key] = ctypes.cast(getattr(lib(), name), ctypes.c_void_p).value
    return e


_marshal = None


def _native():
    """The marshalling module built beside this file (csrc/marshal.cpp): the
    checks, output allocation and C call of the row and QK entry points, on
    torch's C++ tensors.  Raises if it has not been built."""
    global _marshal
    if _marshal is None:
        try:
            from . import _marshal as m
        except ImportError as e:
            raise RuntimeError(f"{_build.marshal_path()} is missing or does not load ({e}): build it first "
                               "(python -c 'import __graft_entry__ as g; g.build()')") from e
        _marshal = m
    return _marshal


def library_path() -> str:
    return _build.LIBRARY


def load(path: str) -> ctypes.CDLL:
    """A build of the library at `path`, with every entry point's C signature
    set.  Raises if the file does not exist."""
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it first (python -c 'import __graft_entry__ as g; g.build()')")
    handle = ctypes.CDLL(path)
    for name, argtypes in _SIGNATURES.items():
        fn = getattr(handle, name)
        fn.argtypes = argtypes
        fn.restype = ctypes.c_int
    handle.rq_status_string.argtypes = [ctypes.c_int]
    handle.rq_status_string.restype = ctypes.c_char_p
    return handle


def lib() -> ctypes.CDLL:
    """The loaded C library.  Raises if it has not been built."""
    global _lib
    if _lib is None:
        with _lock:
            if _lib is None:
                _lib = load(library_path())
    return _lib


def status_string(status: int) -> str:
    return lib().rq_status_string(status).decode()


def _check(status: int, name: str):
    """Map a status code: True on success, False for 'cannot fuse'
    (RQ_ERR_UNSUPPORTED), raise otherwise (ValueError for RQ_ERR_INVALID,
    RuntimeError for RQ_ERR_DEVICE, RQ_ERR_HIP and unknown codes)."""
    if status == RQ_OK:
        return True
    if status == RQ_ERR_UNSUPPORTED:
        return False
    msg = f"{name}: {status_string(status)}"
    if status == RQ_ERR_INVALID:
        raise ValueError(msg)
    raise RuntimeError(msg)


def _status(status: int, name: str):
    """A marshalled call that did not return RQ_OK: None for 'cannot fuse',
    raise for the rest (as _check)."""
    _check(status, name)
    return None



# What the marshalling module's rows(), quantize() and qk() run (csrc/marshal.cpp)
_FP8_TOKEN, _FP8_GROUP, _MXFP4, _FP8_GROUP_TSCALE, _MXFP4_TSCALE, _NORM = range(6)
_QK_BF16, _QK_FP8, _QK_MXFP4 = range(3)


def rmsnorm_quant_fp8_per_token(x, residual, weight, eps: float = 1e-6, *, residual_out=None, q_out=None,
                                scale_out=None, emit_y: bool = False, y_out=None, stream=None):
    """-> (q [M, H] float8_e4m3fn, residual_out [M, H] bf16, scale [M, 1] fp32, y or None), or None."""
    r = _native().rows(_FP8_TOKEN, _entries("rmsnorm_quant_fp8_per_token"), x, residual, weight, eps, 0,
                       residual_out, q_out, scale_out, emit_y, y_out, stream)
    return r if r.__class__ is tuple else _status(r, "rmsnorm_quant_fp8_per_token")


def rmsnorm_quant_fp8_per_group(x, residual, weight, eps: float = 1e-6, group: int = 128, *, residual_out=None,
                                q_out=None, scale_out=None, emit_y: bool = False, y_out=None, stream=None):
    """-> (q [M, H] float8_e4m3fn, residual_out, scale [M, H/group] fp32, y or None), or None."""
    r = _native().rows(_FP8_GROUP, _entries("rmsnorm_quant_fp8_per_group"), x, residual, weight, eps, group,
                       residual_out, q_out, scale_out, emit_y, y_out, stream)
    return r if r.__class__ is tuple else _status(r, "rmsnorm_quant_fp8_per_group")


def rmsnorm_quant_mxfp4(x, residual, weight, eps: float = 1e-6, *, residual_out=None, q_out=None,
                        scale_out=None, emit_y: bool = False, y_out=None, stream=None):
    """-> (q [M, H/2] uint8 packed E2M1, residual_out, scale [M, H/32] uint8 E8M0, y or None), or None."""
    r = _native().rows(_MXFP4, _entries("rmsnorm_quant_mxfp4"), x, residual, weight, eps, 0,
                       residual_out, q_out, scale_out, emit_y, y_out, stream)
    return r if r.__class__ is tuple else _status(r, "rmsnorm_quant_mxfp4")


def rmsnorm_quant_fp8_per_group_tscale(x, residual, weight, eps: float = 1e-6, group: int = 128, *,
                                       residual_out=None, q_out=None, scale_out=None, emit_y: bool = False,
                                       y_out=None, stream=None):
    """Per-group FP8 with column-major scales: scale of row m, group g at scale[g, m].
    scale_out: [H/group, n >= M] fp32 with unit column stride (a view of a wider buffer is fine; its row
    stride is the leading dimension), allocated [H/group, M] when None.
    -> (q [M, H] float8_e4m3fn, residual_out, scale [H/group, >= M] fp32, y or None), or None."""
    r = _native().rows(_FP8_GROUP_TSCALE, _entries("rmsnorm_quant_fp8_per_group_tscale"), x, residual, weight, eps,
                       group, residual_out, q_out, scale_out, emit_y, y_out, stream)
    return r if r.__class__ is tuple else _status(r, "rmsnorm_quant_fp8_per_group_tscale")


def rmsnorm_quant_mxfp4_tscale(x, residual, weight, eps: float = 1e-6, *, residual_out=None, q_out=None,
                               scale_out=None, emit_y: bool = False, y_out=None, stream=None):
    """MXFP4 with column-major E8M0 scales: block b of row m at scale[b, m].
    scale_out: [H/32, n >= M] uint8 with unit column stride, allocated [H/32, M] when None.
    -> (q [M, H/2] uint8 packed E2M1, residual_out, scale [H/32, >= M] uint8, y or None), or None."""
    r = _native().rows(_MXFP4_TSCALE, _entries("rmsnorm_quant_mxfp4_tscale"), x, residual, weight, eps, 0,
                       residual_out, q_out, scale_out, emit_y, y_out, stream)
    return r if r.__class__ is tuple else _status(r, "rmsnorm_quant_mxfp4_tscale")


def qk_gemma_rmsnorm_gate(qg, k, q_w, k_w, num_q_heads: int, num_k_heads: int, head_dim: int,
                          eps: float = 1e-6, *, q_out=None, k_out=None, gate_out=None, stream=None):
    """qg [T, >= 2*Hq*D] interleaved per head as [q | gate]; k [T, >= Hk*D] (row stride allowed); q_w and
    k_w [D] bf16, all bf16 on one device.
    -> (q [T, Hq, D], k [T, Hk, D], gate [T, Hq, D]) contiguous bf16, or None."""
    r = _native().qk(_QK_BF16, _entry("qk_gemma_rmsnorm_gate"), qg, k, q_w, k_w, num_q_heads, num_k_heads,
                     head_dim, eps, q_out, None, k_out, None, gate_out, stream)
    return r if r.__class__ is tuple else _status(r, "qk_gemma_rmsnorm_gate")


def qk_gemma_rmsnorm_gate_fp8(qg, k, q_w, k_w, num_q_heads: int, num_k_heads: int, head_dim: int,
                              eps: float = 1e-6, *, q_out=None, q_scale_out=None, k_out=None, k_scale_out=None,
                              gate_out=None, stream=None):
    """As qk_gemma_rmsnorm_gate, with q and k quantized per head to FP8 E4M3FN (caller code buffers may be
    float8_e4m3fn or uint8, and come back as given).
    -> (q [T, Hq, D] float8_e4m3fn, q_scale [T, Hq] fp32, k [T, Hk, D] float8_e4m3fn, k_scale [T, Hk] fp32,
        gate [T, Hq, D] bf16), or None."""
    r = _native().qk(_QK_FP8, _entry("qk_gemma_rmsnorm_gate_fp8"), qg, k, q_w, k_w, num_q_heads, num_k_heads,
                     head_dim, eps, q_out, q_scale_out, k_out, k_scale_out, gate_out, stream)
    return r if r.__class__ is tuple else _status(r, "qk_gemma_rmsnorm_gate_fp8")


def qk_gemma_rmsnorm_gate_mxfp4(qg, k, q_w, k_w, num_q_heads: int, num_k_heads: int, head_dim: int,
                                eps: float = 1e-6, *, q_out=None, q_scale_out=None, k_out=None, k_scale_out=None,
                                gate_out=None, stream=None):
    """As qk_gemma_rmsnorm_gate, with q and k quantized to MXFP4 (head_dim a multiple of 32).
    -> (q [T, Hq, D/2] uint8 packed E2M1, q_scale [T, Hq, D/32] uint8 E8M0, k [T, Hk, D/2], k_scale [T, Hk, D/32],
        gate [T, Hq, D] bf16), or None."""
    r = _native().qk(_QK_MXFP4, _entry("qk_gemma_rmsnorm_gate_mxfp4"), qg, k, q_w, k_w, num_q_heads, num_k_heads,
                     head_dim, eps, q_out, q_scale_out, k_out, k_scale_out, gate_out, stream)
    return r if r.__class__ is tuple else _status(r, "qk_gemma_rmsnorm_gate_mxfp4")


# ---- the unfused sequence, one launch per step ----

def rmsnorm_residual_bf16(x, residual, weight, eps: float = 1e-6, *, residual_out=None, y_out=None, stream=None):
    """The norm launch of the unfused sequence (rmsnorm_residual_bf16, or
    rmsnorm_residual_f16 for fp16 rows).
    -> (residual_out [M, H], y [M, H]) in the dtype of x, or None."""
    r = _native().rows(_NORM, _entries("rmsnorm_residual"), x, residual, weight, eps, 0, residual_out, None, None,
                       True, y_out, stream)
    return r if r.__class__ is tuple else _status(r, "rmsnorm_residual_bf16")


def quantize_fp8_per_token(y, *, q_out=None, scale_out=None, stream=None):
    """-> (q [M, H] float8_e4m3fn, scale [M, 1] fp32), or None."""
    r = _native().quantize(_FP8_TOKEN, _entries("quantize_fp8_per_token"), y, 0, q_out, scale_out, stream)
    return r if r.__class__ is tuple else _status(r, "quantize_fp8_per_token")


def quantize_fp8_per_group(y, group: int = 128, *, q_out=None, scale_out=None, stream=None):
    """-> (q [M, H] float8_e4m3fn, scale [M, H/group] fp32), or None."""
    r = _native().quantize(_FP8_GROUP, _entries("quantize_fp8_per_group"), y, group, q_out, scale_out, stream)
    return r if r.__class__ is tuple else _status(r, "quantize_fp8_per_group")


def quantize_mxfp4(y, *, q_out=None, scale_out=None, stream=None):
    """-> (q [M, H/2] uint8 packed E2M1, scale [M, H/32] uint8 E8M0), or None."""
    r = _native().quantize(_MXFP4, _entries("quantize_mxfp4"), y, 0, q_out, scale_out, stream)
    return r if r.__class__ is tuple else _status(r, "quantize_mxfp4")


# The fp16 entry points under their C names.  Every function above already
# dispatches on the tensors' dtype (bf16 or fp16), so these are the same
# functions; calling one with bf16 tensors runs the bf16 kernels.
rmsnorm_quant_fp8_per_token_f16 = rmsnorm_quant_fp8_per_token
rmsnorm_quant_fp8_per_group_f16 = rmsnorm_quant_fp8_per_group
rmsnorm_quant_mxfp4_f16 = rmsnorm_quant_mxfp4
rmsnorm_residual_f16 = rmsnorm_residual_bf16
quantize_fp8_per_token_f16 = quantize_fp8_per_token
quantize_fp8_per_group_f16 = quantize_fp8_per_group
quantize_mxfp4_f16 = quantize_mxfp4
rmsnorm_quant_fp8_per_group_tscale_f16 = rmsnorm_quant_fp8_per_group_tscale
rmsnorm_quant_mxfp4_tscale_f16 = rmsnorm_quant_mxfp4_tscale
