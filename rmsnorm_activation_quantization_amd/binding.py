"""Thin ctypes binding of librmsnorm_quant.so (argument marshalling only).

Every entry point has the name of the C function it calls (include/rmsnorm_quant.h).
torch supplies device memory and the current stream; every step of the
computation runs in the library's HIP kernels.  There is no other code path:
if the library is missing (RuntimeError at the first call) or the device is
not an MI355X (RQ_ERR_DEVICE, RuntimeError), calls fail loudly.

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

import torch

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

_ELEMENT_TYPES = (torch.bfloat16, torch.float16)


_FN_CACHE: dict = {}


def _fn(name: str, dtype):
    """The C entry point for an element type: bf16 -> name (rmsnorm_residual_bf16
    for the norm launch), fp16 -> name_f16."""
    key = (name, dtype)
    fn = _FN_CACHE.get(key)
    if fn is None:
        if dtype == torch.float16:
            fn = getattr(lib(), name + "_f16")
        else:
            fn = getattr(lib(), name + ("_bf16" if name == "rmsnorm_residual" else ""))
        _FN_CACHE[key] = fn
    return fn


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


def _ptr(t: torch.Tensor | None) -> int | None:
    return None if t is None else t.data_ptr()


# torch's current stream as a raw handle: the private accessor is ~30x cheaper
# than building a Stream object, which matters for eager decode-sized calls.
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(stream, t: torch.Tensor) -> int:
    if stream is not None:
        return stream.cuda_stream
    if _raw_stream is not None:
        return _raw_stream(t.get_device())
    return torch.cuda.current_stream(t.device).cuda_stream


def _rows(t: torch.Tensor, name: str, dtype=None) -> int:
    """Row stride (elements) of a 2-D bf16 or fp16 CUDA tensor with unit column
    stride (and the given dtype, when one is given)."""
    if t.dim() != 2 or t.dtype not in _ELEMENT_TYPES or not t.is_cuda:
        raise ValueError(f"{name} must be a 2-D bfloat16 or float16 CUDA tensor")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must have the dtype of x ({dtype})")
    if t.shape[1] > 1 and t.stride(1) != 1:
        raise ValueError(f"{name} must have unit column stride")
    return t.stride(0) if t.shape[0] > 1 else t.shape[1]


def _same_device(like: torch.Tensor, **tensors) -> None:
    """Every given tensor (None skipped) on the device of `like`: the kernels
    dereference every pointer on that device, so a host tensor or one on
    another GPU is refused here."""
    for name, t in tensors.items():
        if t is not None and t.device != like.device:
            raise ValueError(f"{name} is on {t.device}; every tensor must be on {like.device}")


def _row_outputs(x, residual, weight, residual_out, y_out, emit_y):
    """Checks the row inputs (one element type for all, one device) and
    allocates the missing row outputs in that type."""
    M, H = x.shape
    dt = x.dtype
    if residual.shape != (M, H) or weight.shape != (H,) or residual.dtype != dt or weight.dtype != dt:
        raise ValueError(f"residual must be [M, H] and weight [H], both {dt} like x")
    if not weight.is_contiguous():
        raise ValueError("weight must be contiguous")
    _same_device(x, residual=residual, weight=weight, residual_out=residual_out, y_out=y_out)
    if residual_out is None:
        residual_out = torch.empty((M, H), dtype=dt, device=x.device)
    if y_out is None and emit_y:
        y_out = torch.empty((M, H), dtype=dt, device=x.device)
    for name, t in (("residual_out", residual_out), ("y_out", y_out)):
        if t is not None and (t.shape != (M, H) or t.dtype != dt or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous [M, H] {dt} tensor")
    return M, H, residual_out, y_out


def _out(t, shape, dtypes, name, like):
    """A caller-supplied output: the exact shape, one of the dtypes, contiguous,
    on the device of `like`.  The library cannot see buffer sizes, so a wrong
    output tensor is refused here rather than written past its end."""
    if tuple(t.shape) != tuple(shape) or t.dtype not in dtypes or not t.is_contiguous() or t.device != like.device:
        raise ValueError(f"{name} must be a contiguous {list(shape)} {dtypes[0]} tensor on {like.device}")
    return t


_CODES8 = (torch.uint8, torch.float8_e4m3fn)


def rmsnorm_quant_fp8_per_token(x, residual, weight, eps: float = 1e-6, *, residual_out=None, q_out=None,
                                scale_out=None, emit_y: bool = False, y_out=None, stream=None):
    """-> (q [M, H] float8_e4m3fn, residual_out [M, H] bf16, scale [M, 1] fp32, y or None), or None."""
    ldx, ldr = _rows(x, "x"), _rows(residual, "residual", x.dtype)
    M, H, residual_out, y_out = _row_outputs(x, residual, weight, residual_out, y_out, emit_y)
    q_out = torch.empty((M, H), dtype=torch.uint8, device=x.device) if q_out is None else \
        _out(q_out, (M, H), _CODES8, "q_out", x)
    if scale_out is None:
        scale_out = torch.empty((M,), dtype=torch.float32, device=x.device)
    elif tuple(scale_out.shape) not in ((M,), (M, 1)):
        raise ValueError(f"scale_out must be a contiguous [{M}] or [{M}, 1] float32 tensor")
    else:
        _out(scale_out, scale_out.shape, (torch.float32,), "scale_out", x)
    st = _fn("rmsnorm_quant_fp8_per_token", x.dtype)(
        _ptr(x), ldx, _ptr(residual), ldr, _ptr(weight), M, H, eps, _ptr(residual_out), _ptr(q_out),
        _ptr(scale_out), _ptr(y_out), _stream(stream, x))
    if not _check(st, "rmsnorm_quant_fp8_per_token"):
        return None
    return q_out.view(torch.float8_e4m3fn), residual_out, scale_out.view(M, 1), y_out


def rmsnorm_quant_fp8_per_group(x, residual, weight, eps: float = 1e-6, group: int = 128, *, residual_out=None,
                                q_out=None, scale_out=None, emit_y: bool = False, y_out=None, stream=None):
    """-> (q [M, H] float8_e4m3fn, residual_out, scale [M, H/group] fp32, y or None), or None."""
    ldx, ldr = _rows(x, "x"), _rows(residual, "residual", x.dtype)
    M, H, residual_out, y_out = _row_outputs(x, residual, weight, residual_out, y_out, emit_y)
    G = max(H // group, 1) if group > 0 else 1
    q_out = torch.empty((M, H), dtype=torch.uint8, device=x.device) if q_out is None else \
        _out(q_out, (M, H), _CODES8, "q_out", x)
    scale_out = torch.empty((M, G), dtype=torch.float32, device=x.device) if scale_out is None else \
        _out(scale_out, (M, G), (torch.float32,), "scale_out", x)
    st = _fn("rmsnorm_quant_fp8_per_group", x.dtype)(
        _ptr(x), ldx, _ptr(residual), ldr, _ptr(weight), M, H, eps, group, _ptr(residual_out), _ptr(q_out),
        _ptr(scale_out), _ptr(y_out), _stream(stream, x))
    if not _check(st, "rmsnorm_quant_fp8_per_group"):
        return None
    return q_out.view(torch.float8_e4m3fn), residual_out, scale_out, y_out


def rmsnorm_quant_mxfp4(x, residual, weight, eps: float = 1e-6, *, residual_out=None, q_out=None,
                        scale_out=None, emit_y: bool = False, y_out=None, stream=None):
    """-> (q [M, H/2] uint8 packed E2M1, residual_out, scale [M, H/32] uint8 E8M0, y or None), or None."""
    ldx, ldr = _rows(x, "x"), _rows(residual, "residual", x.dtype)
    M, H, residual_out, y_out = _row_outputs(x, residual, weight, residual_out, y_out, emit_y)
    q_out = torch.empty((M, H // 2), dtype=torch.uint8, device=x.device) if q_out is None else \
        _out(q_out, (M, H // 2), (torch.uint8,), "q_out", x)
    scale_out = torch.empty((M, max(H // 32, 1)), dtype=torch.uint8, device=x.device) if scale_out is None else \
        _out(scale_out, (M, max(H // 32, 1)), (torch.uint8,), "scale_out", x)
    st = _fn("rmsnorm_quant_mxfp4", x.dtype)(
        _ptr(x), ldx, _ptr(residual), ldr, _ptr(weight), M, H, eps, _ptr(residual_out), _ptr(q_out),
        _ptr(scale_out), _ptr(y_out), _stream(stream, x))
    if not _check(st, "rmsnorm_quant_mxfp4"):
        return None
    return q_out, residual_out, scale_out, y_out


def _tscale_out(scale_out, rows, M, dtype, x):
    """Column-major scales: a [rows, n >= M] tensor with unit column stride
    (a view of a wider buffer is fine); its row stride is ld_scale."""
    if scale_out is None:
        scale_out = torch.empty((rows, max(M, 1)), dtype=dtype, device=x.device)
    if (scale_out.dim() != 2 or scale_out.shape[0] != rows or scale_out.shape[1] < M or scale_out.dtype != dtype
            or (scale_out.shape[1] > 1 and scale_out.stride(1) != 1) or scale_out.device != x.device):
        raise ValueError(f"scale_out must be a [{rows}, >= {M}] {dtype} tensor with unit column stride")
    ld = scale_out.stride(0) if rows > 1 else max(scale_out.shape[1], 1)
    return scale_out, ld


def rmsnorm_quant_fp8_per_group_tscale(x, residual, weight, eps: float = 1e-6, group: int = 128, *,
                                       residual_out=None, q_out=None, scale_out=None, emit_y: bool = False,
                                       y_out=None, stream=None):
    """Per-group FP8 with column-major scales: scale of row m, group g at scale[g, m].
    -> (q [M, H] float8_e4m3fn, residual_out, scale [H/group, >= M] fp32, y or None), or None."""
    ldx, ldr = _rows(x, "x"), _rows(residual, "residual", x.dtype)
    M, H, residual_out, y_out = _row_outputs(x, residual, weight, residual_out, y_out, emit_y)
    G = max(H // group, 1) if group > 0 else 1
    q_out = torch.empty((M, H), dtype=torch.uint8, device=x.device) if q_out is None else \
        _out(q_out, (M, H), _CODES8, "q_out", x)
    scale_out, ld = _tscale_out(scale_out, G, M, torch.float32, x)
    st = _fn("rmsnorm_quant_fp8_per_group_tscale", x.dtype)(
        _ptr(x), ldx, _ptr(residual), ldr, _ptr(weight), M, H, eps, group, _ptr(residual_out), _ptr(q_out),
        _ptr(scale_out), ld, _ptr(y_out), _stream(stream, x))
    if not _check(st, "rmsnorm_quant_fp8_per_group_tscale"):
        return None
    return q_out.view(torch.float8_e4m3fn), residual_out, scale_out, y_out


def rmsnorm_quant_mxfp4_tscale(x, residual, weight, eps: float = 1e-6, *, residual_out=None, q_out=None,
                               scale_out=None, emit_y: bool = False, y_out=None, stream=None):
    """MXFP4 with column-major E8M0 scales: block b of row m at scale[b, m].
    -> (q [M, H/2] uint8 packed E2M1, residual_out, scale [H/32, >= M] uint8, y or None), or None."""
    ldx, ldr = _rows(x, "x"), _rows(residual, "residual", x.dtype)
    M, H, residual_out, y_out = _row_outputs(x, residual, weight, residual_out, y_out, emit_y)
    q_out = torch.empty((M, H // 2), dtype=torch.uint8, device=x.device) if q_out is None else \
        _out(q_out, (M, H // 2), (torch.uint8,), "q_out", x)
    scale_out, ld = _tscale_out(scale_out, max(H // 32, 1), M, torch.uint8, x)
    st = _fn("rmsnorm_quant_mxfp4_tscale", x.dtype)(
        _ptr(x), ldx, _ptr(residual), ldr, _ptr(weight), M, H, eps, _ptr(residual_out), _ptr(q_out),
        _ptr(scale_out), ld, _ptr(y_out), _stream(stream, x))
    if not _check(st, "rmsnorm_quant_mxfp4_tscale"):
        return None
    return q_out, residual_out, scale_out, y_out


def _qk_inputs(qg, k, q_w, k_w, head_dim: int):
    """Checks of the QK inputs (bf16 only, one device) -> (ld_qg, ld_k, T)."""
    ld_qg, ld_k = _rows(qg, "qg", torch.bfloat16), _rows(k, "k", torch.bfloat16)
    T = qg.shape[0]
    if k.shape[0] != T:
        raise ValueError("qg and k must have the same number of tokens")
    for name, w in (("q_w", q_w), ("k_w", k_w)):
        if w.shape != (head_dim,) or w.dtype != torch.bfloat16 or not w.is_contiguous():
            raise ValueError(f"{name} must be a contiguous [head_dim] bfloat16 tensor")
    _same_device(qg, k=k, q_w=q_w, k_w=k_w)
    return ld_qg, ld_k, T


def qk_gemma_rmsnorm_gate(qg, k, q_w, k_w, num_q_heads: int, num_k_heads: int, head_dim: int,
                          eps: float = 1e-6, *, q_out=None, k_out=None, gate_out=None, stream=None):
    """qg [T, >= 2*Hq*D] interleaved per head as [q | gate]; k [T, >= Hk*D] (row stride allowed).
    -> (q [T, Hq, D], k [T, Hk, D], gate [T, Hq, D]) contiguous bf16, or None."""
    ld_qg, ld_k, T = _qk_inputs(qg, k, q_w, k_w, head_dim)
    Hq, Hk, D = num_q_heads, num_k_heads, head_dim
    dev = qg.device
    q_out = torch.empty((T, Hq, D), dtype=torch.bfloat16, device=dev) if q_out is None else q_out
    k_out = torch.empty((T, Hk, D), dtype=torch.bfloat16, device=dev) if k_out is None else k_out
    gate_out = torch.empty((T, Hq, D), dtype=torch.bfloat16, device=dev) if gate_out is None else gate_out
    for name, t, h in (("q_out", q_out, Hq), ("k_out", k_out, Hk), ("gate_out", gate_out, Hq)):
        if t.shape != (T, h, D) or t.dtype != torch.bfloat16 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous [T, heads, head_dim] bfloat16 tensor")
    _same_device(qg, q_out=q_out, k_out=k_out, gate_out=gate_out)
    st = lib().qk_gemma_rmsnorm_gate(
        _ptr(qg), ld_qg, _ptr(k), ld_k, _ptr(q_w), _ptr(k_w), T, Hq, Hk, D, eps, _ptr(q_out), _ptr(k_out),
        _ptr(gate_out), _stream(stream, qg))
    if not _check(st, "qk_gemma_rmsnorm_gate"):
        return None
    return q_out, k_out, gate_out


def qk_gemma_rmsnorm_gate_fp8(qg, k, q_w, k_w, num_q_heads: int, num_k_heads: int, head_dim: int,
                              eps: float = 1e-6, *, q_out=None, q_scale_out=None, k_out=None, k_scale_out=None,
                              gate_out=None, stream=None):
    """As qk_gemma_rmsnorm_gate, with q and k quantized per head to FP8 E4M3FN.
    -> (q [T, Hq, D] float8_e4m3fn, q_scale [T, Hq] fp32, k [T, Hk, D] float8_e4m3fn, k_scale [T, Hk] fp32,
        gate [T, Hq, D] bf16), or None."""
    ld_qg, ld_k, T = _qk_inputs(qg, k, q_w, k_w, head_dim)
    Hq, Hk, D = num_q_heads, num_k_heads, head_dim
    dev = qg.device
    fp8 = torch.float8_e4m3fn
    q_out = torch.empty((T, Hq, D), dtype=fp8, device=dev) if q_out is None else q_out
    k_out = torch.empty((T, Hk, D), dtype=fp8, device=dev) if k_out is None else k_out
    q_scale_out = torch.empty((T, Hq), dtype=torch.float32, device=dev) if q_scale_out is None else q_scale_out
    k_scale_out = torch.empty((T, Hk), dtype=torch.float32, device=dev) if k_scale_out is None else k_scale_out
    gate_out = torch.empty((T, Hq, D), dtype=torch.bfloat16, device=dev) if gate_out is None else gate_out
    for name, t, shape, dts in (("q_out", q_out, (T, Hq, D), (fp8, torch.uint8)),
                                ("k_out", k_out, (T, Hk, D), (fp8, torch.uint8)),
                                ("q_scale_out", q_scale_out, (T, Hq), (torch.float32,)),
                                ("k_scale_out", k_scale_out, (T, Hk), (torch.float32,)),
                                ("gate_out", gate_out, (T, Hq, D), (torch.bfloat16,))):
        if tuple(t.shape) != shape or t.dtype not in dts or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous {list(shape)} tensor of {dts[0]}")
    _same_device(qg, q_out=q_out, k_out=k_out, q_scale_out=q_scale_out, k_scale_out=k_scale_out, gate_out=gate_out)
    st = lib().qk_gemma_rmsnorm_gate_fp8(
        _ptr(qg), ld_qg, _ptr(k), ld_k, _ptr(q_w), _ptr(k_w), T, Hq, Hk, D, eps, _ptr(q_out), _ptr(q_scale_out),
        _ptr(k_out), _ptr(k_scale_out), _ptr(gate_out), _stream(stream, qg))
    if not _check(st, "qk_gemma_rmsnorm_gate_fp8"):
        return None
    return q_out, q_scale_out, k_out, k_scale_out, gate_out


def qk_gemma_rmsnorm_gate_mxfp4(qg, k, q_w, k_w, num_q_heads: int, num_k_heads: int, head_dim: int,
                                eps: float = 1e-6, *, q_out=None, q_scale_out=None, k_out=None, k_scale_out=None,
                                gate_out=None, stream=None):
    """As qk_gemma_rmsnorm_gate, with q and k quantized to MXFP4 (head_dim a multiple of 32).
    -> (q [T, Hq, D/2] uint8 packed E2M1, q_scale [T, Hq, D/32] uint8 E8M0, k [T, Hk, D/2], k_scale [T, Hk, D/32],
        gate [T, Hq, D] bf16), or None."""
    ld_qg, ld_k, T = _qk_inputs(qg, k, q_w, k_w, head_dim)
    Hq, Hk, D = num_q_heads, num_k_heads, head_dim
    dev = qg.device
    u8 = torch.uint8
    shapes = {"q_out": (T, Hq, D // 2), "q_scale_out": (T, Hq, max(D // 32, 1)), "k_out": (T, Hk, D // 2),
              "k_scale_out": (T, Hk, max(D // 32, 1)), "gate_out": (T, Hq, D)}
    given = {"q_out": q_out, "q_scale_out": q_scale_out, "k_out": k_out, "k_scale_out": k_scale_out,
             "gate_out": gate_out}
    outs = {}
    for name, shape in shapes.items():
        dt = torch.bfloat16 if name == "gate_out" else u8
        t = given[name]
        outs[name] = torch.empty(shape, dtype=dt, device=dev) if t is None else _out(t, shape, (dt,), name, qg)
    st = lib().qk_gemma_rmsnorm_gate_mxfp4(
        _ptr(qg), ld_qg, _ptr(k), ld_k, _ptr(q_w), _ptr(k_w), T, Hq, Hk, D, eps, _ptr(outs["q_out"]),
        _ptr(outs["q_scale_out"]), _ptr(outs["k_out"]), _ptr(outs["k_scale_out"]), _ptr(outs["gate_out"]),
        _stream(stream, qg))
    if not _check(st, "qk_gemma_rmsnorm_gate_mxfp4"):
        return None
    return outs["q_out"], outs["q_scale_out"], outs["k_out"], outs["k_scale_out"], outs["gate_out"]


# ---- the unfused sequence, one launch per step ----

def rmsnorm_residual_bf16(x, residual, weight, eps: float = 1e-6, *, residual_out=None, y_out=None, stream=None):
    """-> (residual_out [M, H] bf16, y [M, H] bf16), or None."""
    ldx, ldr = _rows(x, "x"), _rows(residual, "residual", x.dtype)
    M, H, residual_out, y_out = _row_outputs(x, residual, weight, residual_out, y_out, True)
    st = _fn("rmsnorm_residual", x.dtype)(_ptr(x), ldx, _ptr(residual), ldr, _ptr(weight), M, H, eps,
                                     _ptr(residual_out), _ptr(y_out), _stream(stream, x))
    if not _check(st, "rmsnorm_residual_bf16"):
        return None
    return residual_out, y_out


def _quant_input(y):
    ldy = _rows(y, "y")
    return ldy, y.shape[0], y.shape[1]


def quantize_fp8_per_token(y, *, q_out=None, scale_out=None, stream=None):
    """-> (q [M, H] float8_e4m3fn, scale [M, 1] fp32), or None."""
    ldy, M, H = _quant_input(y)
    q_out = torch.empty((M, H), dtype=torch.uint8, device=y.device) if q_out is None else \
        _out(q_out, (M, H), _CODES8, "q_out", y)
    if scale_out is None:
        scale_out = torch.empty((M,), dtype=torch.float32, device=y.device)
    elif tuple(scale_out.shape) not in ((M,), (M, 1)):
        raise ValueError(f"scale_out must be a contiguous [{M}] or [{M}, 1] float32 tensor")
    else:
        _out(scale_out, scale_out.shape, (torch.float32,), "scale_out", y)
    st = _fn("quantize_fp8_per_token", y.dtype)(_ptr(y), ldy, M, H, _ptr(q_out), _ptr(scale_out), _stream(stream, y))
    if not _check(st, "quantize_fp8_per_token"):
        return None
    return q_out.view(torch.float8_e4m3fn), scale_out.view(M, 1)


def quantize_fp8_per_group(y, group: int = 128, *, q_out=None, scale_out=None, stream=None):
    """-> (q [M, H] float8_e4m3fn, scale [M, H/group] fp32), or None."""
    ldy, M, H = _quant_input(y)
    G = max(H // group, 1) if group > 0 else 1
    q_out = torch.empty((M, H), dtype=torch.uint8, device=y.device) if q_out is None else \
        _out(q_out, (M, H), _CODES8, "q_out", y)
    scale_out = torch.empty((M, G), dtype=torch.float32, device=y.device) if scale_out is None else \
        _out(scale_out, (M, G), (torch.float32,), "scale_out", y)
    st = _fn("quantize_fp8_per_group", y.dtype)(_ptr(y), ldy, M, H, group, _ptr(q_out), _ptr(scale_out), _stream(stream, y))
    if not _check(st, "quantize_fp8_per_group"):
        return None
    return q_out.view(torch.float8_e4m3fn), scale_out


def quantize_mxfp4(y, *, q_out=None, scale_out=None, stream=None):
    """-> (q [M, H/2] uint8 packed E2M1, scale [M, H/32] uint8 E8M0), or None."""
    ldy, M, H = _quant_input(y)
    q_out = torch.empty((M, H // 2), dtype=torch.uint8, device=y.device) if q_out is None else \
        _out(q_out, (M, H // 2), (torch.uint8,), "q_out", y)
    scale_out = torch.empty((M, max(H // 32, 1)), dtype=torch.uint8, device=y.device) if scale_out is None else \
        _out(scale_out, (M, max(H // 32, 1)), (torch.uint8,), "scale_out", y)
    st = _fn("quantize_mxfp4", y.dtype)(_ptr(y), ldy, M, H, _ptr(q_out), _ptr(scale_out), _stream(stream, y))
    if not _check(st, "quantize_mxfp4"):
        return None
    return q_out, scale_out


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
