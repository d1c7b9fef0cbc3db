"""CPU oracle for the fused residual-add -> RMSNorm -> quantization step.

TEST INFRASTRUCTURE ONLY.  This package builds and loads ``librq_oracle.so``
(plain C++ in ``rq_oracle.cpp``, fp64 arithmetic) and wraps it for numpy.  Only
the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py``
may import it.  The HIP library never imports, links or calls anything here,
and this package imports nothing from the HIP library.

Every function's definition is documented in ``rq_oracle.h`` with the page and
section it follows.  Parity pins for each function live in
``tests/test_oracle_*.py``.
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_DIR = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_DIR, "rq_oracle.cpp")
LIBRARY = os.path.join(_DIR, "librq_oracle.so")

# No fast-math and no FMA contraction: each C++ operation rounds exactly once.
CXXFLAGS = ["-O2", "-std=c++17", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math"]


def build(source: str = SOURCE, output: str = LIBRARY) -> str:
    """Compile the oracle with g++ into a shared library and return its path."""
    tmp = output + ".tmp"
    subprocess.run(["g++", *CXXFLAGS, "-I", os.path.dirname(source), source, "-o", tmp],
                   check=True)
    os.replace(tmp, output)
    return output


_u16p = ctypes.POINTER(ctypes.c_uint16)
_u8p = ctypes.POINTER(ctypes.c_uint8)
_f32p = ctypes.POINTER(ctypes.c_float)
_i64 = ctypes.c_int64


def _ptr(a: np.ndarray | None, ctype):
    if a is None:
        return ctypes.cast(None, ctype)
    return a.ctypes.data_as(ctype)


def _rows(a: np.ndarray) -> tuple[np.ndarray, int]:
    """A 2-D uint16 array whose rows may be strided; returns (array, ld)."""
    a = np.asarray(a)
    assert a.dtype == np.uint16 and a.ndim == 2
    if a.strides[1] != 2 or a.strides[0] % 2:
        a = np.ascontiguousarray(a)
    return a, a.strides[0] // 2 if a.shape[0] > 0 else a.shape[1]


class Oracle:
    """numpy front end of librq_oracle.so.  bf16 and fp16 arrays are uint16 bit
    patterns; the row functions take dtype="bf16" (default) or "fp16"."""

    def __init__(self, path: str = LIBRARY):
        if not os.path.exists(path):
            build(output=path)
        lib = ctypes.CDLL(path)
        self.lib = lib
        lib.rq_ref_f64_from_bf16.argtypes = [ctypes.c_uint16]
        lib.rq_ref_f64_from_bf16.restype = ctypes.c_double
        lib.rq_ref_bf16_from_f64.argtypes = [ctypes.c_double]
        lib.rq_ref_bf16_from_f64.restype = ctypes.c_uint16
        lib.rq_ref_e4m3fn_from_f64.argtypes = [ctypes.c_double]
        lib.rq_ref_e4m3fn_from_f64.restype = ctypes.c_uint8
        lib.rq_ref_f64_from_e4m3fn.argtypes = [ctypes.c_uint8]
        lib.rq_ref_f64_from_e4m3fn.restype = ctypes.c_double
        lib.rq_ref_e2m1_from_f64.argtypes = [ctypes.c_double]
        lib.rq_ref_e2m1_from_f64.restype = ctypes.c_uint8
        lib.rq_ref_f64_from_e2m1.argtypes = [ctypes.c_uint8]
        lib.rq_ref_f64_from_e2m1.restype = ctypes.c_double
        lib.rq_ref_e8m0_from_amax.argtypes = [ctypes.c_double]
        lib.rq_ref_e8m0_from_amax.restype = ctypes.c_uint8
        lib.rq_ref_f64_from_e8m0.argtypes = [ctypes.c_uint8]
        lib.rq_ref_f64_from_e8m0.restype = ctypes.c_double
        lib.rq_ref_f64_from_f16.argtypes = [ctypes.c_uint16]
        lib.rq_ref_f64_from_f16.restype = ctypes.c_double
        lib.rq_ref_f16_from_f64.argtypes = [ctypes.c_double]
        lib.rq_ref_f16_from_f64.restype = ctypes.c_uint16
        row_args = [_u16p, _i64, _u16p, _i64, _u16p, _i64, _i64, ctypes.c_float]
        for sfx in ("", "_f16"):
            getattr(lib, "rq_ref_rmsnorm_quant_fp8_per_token" + sfx).argtypes = row_args + [_u16p, _u8p, _f32p, _u16p]
            getattr(lib, "rq_ref_rmsnorm_quant_fp8_per_group" + sfx).argtypes = \
                row_args + [_i64, _u16p, _u8p, _f32p, _u16p]
            getattr(lib, "rq_ref_rmsnorm_quant_mxfp4" + sfx).argtypes = row_args + [_u16p, _u8p, _u8p, _u16p]
            getattr(lib, "rq_ref_quantize_fp8" + sfx).argtypes = [_u16p, _i64, _i64, _i64, _u8p, _f32p]
            getattr(lib, "rq_ref_quantize_mxfp4" + sfx).argtypes = [_u16p, _i64, _i64, _u8p, _u8p]
        for sfx in ("", "_f16"):
            fn = getattr(lib, "rq_ref_rmsnorm_quant_fp8_per_group_tscale" + sfx)
            fn.argtypes = row_args + [_i64, _u16p, _u8p, _f32p, _i64, _u16p]
            fn.restype = ctypes.c_int
            fn = getattr(lib, "rq_ref_rmsnorm_quant_mxfp4_tscale" + sfx)
            fn.argtypes = row_args + [_u16p, _u8p, _u8p, _i64, _u16p]
            fn.restype = ctypes.c_int
        lib.rq_ref_qk_gemma_rmsnorm_gate.argtypes = [
            _u16p, _i64, _u16p, _i64, _u16p, _u16p, _i64, _i64, _i64, _i64, ctypes.c_float,
            _u16p, _u16p, _u16p]
        for name in ("rq_ref_quantize_fp8", "rq_ref_quantize_mxfp4",
                     "rq_ref_rmsnorm_quant_fp8_per_token", "rq_ref_rmsnorm_quant_fp8_per_group",
                     "rq_ref_rmsnorm_quant_mxfp4"):
            getattr(lib, name).restype = ctypes.c_int
            getattr(lib, name + "_f16").restype = ctypes.c_int
        lib.rq_ref_qk_gemma_rmsnorm_gate.restype = ctypes.c_int
        lib.rq_ref_qk_gemma_rmsnorm_gate_fp8.argtypes = [
            _u16p, _i64, _u16p, _i64, _u16p, _u16p, _i64, _i64, _i64, _i64, ctypes.c_float,
            _u8p, _f32p, _u8p, _f32p, _u16p]
        lib.rq_ref_qk_gemma_rmsnorm_gate_fp8.restype = ctypes.c_int
        lib.rq_ref_qk_gemma_rmsnorm_gate_mxfp4.argtypes = [
            _u16p, _i64, _u16p, _i64, _u16p, _u16p, _i64, _i64, _i64, _i64, ctypes.c_float,
            _u8p, _u8p, _u8p, _u8p, _u16p]
        lib.rq_ref_qk_gemma_rmsnorm_gate_mxfp4.restype = ctypes.c_int

    def _fn(self, name, dtype):
        if dtype not in ("bf16", "fp16"):
            raise ValueError(f"unknown element type {dtype!r}")
        return getattr(self.lib, name + ("_f16" if dtype == "fp16" else ""))

    # ---- scalar format functions (element-wise over arrays) ----
    def bf16_value(self, bits) -> np.ndarray:
        with np.errstate(invalid="ignore"):
            return np.vectorize(self.lib.rq_ref_f64_from_bf16, otypes=[np.float64])(
                np.asarray(bits, dtype=np.uint16))

    def bf16_round(self, v) -> np.ndarray:
        return np.vectorize(self.lib.rq_ref_bf16_from_f64, otypes=[np.uint16])(
            np.asarray(v, dtype=np.float64))

    def f16_value(self, bits) -> np.ndarray:
        with np.errstate(invalid="ignore"):
            return np.vectorize(self.lib.rq_ref_f64_from_f16, otypes=[np.float64])(
                np.asarray(bits, dtype=np.uint16))

    def f16_round(self, v) -> np.ndarray:
        return np.vectorize(self.lib.rq_ref_f16_from_f64, otypes=[np.uint16])(
            np.asarray(v, dtype=np.float64))

    def e4m3fn(self, v) -> np.ndarray:
        return np.vectorize(self.lib.rq_ref_e4m3fn_from_f64, otypes=[np.uint8])(
            np.asarray(v, dtype=np.float64))

    def e4m3fn_value(self, c) -> np.ndarray:
        return np.vectorize(self.lib.rq_ref_f64_from_e4m3fn, otypes=[np.float64])(
            np.asarray(c, dtype=np.uint8))

    def e2m1(self, v) -> np.ndarray:
        return np.vectorize(self.lib.rq_ref_e2m1_from_f64, otypes=[np.uint8])(
            np.asarray(v, dtype=np.float64))

    def e2m1_value(self, c) -> np.ndarray:
        return np.vectorize(self.lib.rq_ref_f64_from_e2m1, otypes=[np.float64])(
            np.asarray(c, dtype=np.uint8))

    def e8m0(self, amax) -> np.ndarray:
        return np.vectorize(self.lib.rq_ref_e8m0_from_amax, otypes=[np.uint8])(
            np.asarray(amax, dtype=np.float64))

    def e8m0_value(self, b) -> np.ndarray:
        return np.vectorize(self.lib.rq_ref_f64_from_e8m0, otypes=[np.float64])(
            np.asarray(b, dtype=np.uint8))

    # ---- the fused step ----
    def _row_inputs(self, x, residual, weight):
        x, ldx = _rows(x)
        residual, ldr = _rows(residual)
        weight = np.ascontiguousarray(weight, dtype=np.uint16)
        M, H = x.shape
        assert residual.shape == (M, H) and weight.shape == (H,)
        return x, ldx, residual, ldr, weight, M, H

    def fp8_per_token(self, x, residual, weight, eps, emit_y=False, dtype="bf16") -> dict:
        x, ldx, residual, ldr, weight, M, H = self._row_inputs(x, residual, weight)
        out = dict(residual_out=np.zeros((M, H), np.uint16), q=np.zeros((M, H), np.uint8),
                   scale=np.zeros((M,), np.float32),
                   y=np.zeros((M, H), np.uint16) if emit_y else None)
        rc = self._fn("rq_ref_rmsnorm_quant_fp8_per_token", dtype)(
            _ptr(x, _u16p), ldx, _ptr(residual, _u16p), ldr, _ptr(weight, _u16p), M, H, eps,
            _ptr(out["residual_out"], _u16p), _ptr(out["q"], _u8p), _ptr(out["scale"], _f32p),
            _ptr(out["y"], _u16p))
        if rc != 0:
            raise ValueError("oracle rejected the arguments")
        return out

    def fp8_per_group(self, x, residual, weight, eps, group, emit_y=False, dtype="bf16") -> dict:
        x, ldx, residual, ldr, weight, M, H = self._row_inputs(x, residual, weight)
        G = H // group if group > 0 else 0
        out = dict(residual_out=np.zeros((M, H), np.uint16), q=np.zeros((M, H), np.uint8),
                   scale=np.zeros((M, G), np.float32),
                   y=np.zeros((M, H), np.uint16) if emit_y else None)
        rc = self._fn("rq_ref_rmsnorm_quant_fp8_per_group", dtype)(
            _ptr(x, _u16p), ldx, _ptr(residual, _u16p), ldr, _ptr(weight, _u16p), M, H, eps,
            group, _ptr(out["residual_out"], _u16p), _ptr(out["q"], _u8p),
            _ptr(out["scale"], _f32p), _ptr(out["y"], _u16p))
        if rc != 0:
            raise ValueError("oracle rejected the arguments")
        return out

    def mxfp4(self, x, residual, weight, eps, emit_y=False, dtype="bf16") -> dict:
        x, ldx, residual, ldr, weight, M, H = self._row_inputs(x, residual, weight)
        out = dict(residual_out=np.zeros((M, H), np.uint16), q=np.zeros((M, H // 2), np.uint8),
                   scale=np.zeros((M, H // 32), np.uint8),
                   y=np.zeros((M, H), np.uint16) if emit_y else None)
        rc = self._fn("rq_ref_rmsnorm_quant_mxfp4", dtype)(
            _ptr(x, _u16p), ldx, _ptr(residual, _u16p), ldr, _ptr(weight, _u16p), M, H, eps,
            _ptr(out["residual_out"], _u16p), _ptr(out["q"], _u8p), _ptr(out["scale"], _u8p),
            _ptr(out["y"], _u16p))
        if rc != 0:
            raise ValueError("oracle rejected the arguments")
        return out

    # ---- transposed scales: scale (m, g) at [g, m] of a [G, ld_scale] array ----
    def fp8_per_group_tscale(self, x, residual, weight, eps, group, ld_scale=None, emit_y=False,
                             dtype="bf16") -> dict:
        x, ldx, residual, ldr, weight, M, H = self._row_inputs(x, residual, weight)
        G = H // group if group > 0 else 0
        ld = M if ld_scale is None else ld_scale
        out = dict(residual_out=np.zeros((M, H), np.uint16), q=np.zeros((M, H), np.uint8),
                   scale=np.full((max(G, 1), max(ld, 1)), -1.0, np.float32),
                   y=np.zeros((M, H), np.uint16) if emit_y else None)
        rc = self._fn("rq_ref_rmsnorm_quant_fp8_per_group_tscale", dtype)(
            _ptr(x, _u16p), ldx, _ptr(residual, _u16p), ldr, _ptr(weight, _u16p), M, H, eps,
            group, _ptr(out["residual_out"], _u16p), _ptr(out["q"], _u8p),
            _ptr(out["scale"], _f32p), ld, _ptr(out["y"], _u16p))
        if rc != 0:
            raise ValueError("oracle rejected the arguments")
        return out

    def mxfp4_tscale(self, x, residual, weight, eps, ld_scale=None, emit_y=False, dtype="bf16") -> dict:
        x, ldx, residual, ldr, weight, M, H = self._row_inputs(x, residual, weight)
        ld = M if ld_scale is None else ld_scale
        out = dict(residual_out=np.zeros((M, H), np.uint16), q=np.zeros((M, H // 2), np.uint8),
                   scale=np.full((max(H // 32, 1), max(ld, 1)), 0xAB, np.uint8),
                   y=np.zeros((M, H), np.uint16) if emit_y else None)
        rc = self._fn("rq_ref_rmsnorm_quant_mxfp4_tscale", dtype)(
            _ptr(x, _u16p), ldx, _ptr(residual, _u16p), ldr, _ptr(weight, _u16p), M, H, eps,
            _ptr(out["residual_out"], _u16p), _ptr(out["q"], _u8p), _ptr(out["scale"], _u8p), ld,
            _ptr(out["y"], _u16p))
        if rc != 0:
            raise ValueError("oracle rejected the arguments")
        return out

    # ---- the quantize step alone ----
    def quantize_fp8(self, y, group=None, dtype="bf16") -> dict:
        y = np.ascontiguousarray(y, dtype=np.uint16)
        M, H = y.shape
        group = H if group is None else group
        out = dict(q=np.zeros((M, H), np.uint8), scale=np.zeros((M, H // group), np.float32))
        rc = self._fn("rq_ref_quantize_fp8", dtype)(_ptr(y, _u16p), M, H, group, _ptr(out["q"], _u8p),
                                          _ptr(out["scale"], _f32p))
        if rc != 0:
            raise ValueError("oracle rejected the arguments")
        return out

    def quantize_mxfp4(self, y, dtype="bf16") -> dict:
        y = np.ascontiguousarray(y, dtype=np.uint16)
        M, H = y.shape
        out = dict(q=np.zeros((M, H // 2), np.uint8), scale=np.zeros((M, H // 32), np.uint8))
        rc = self._fn("rq_ref_quantize_mxfp4", dtype)(_ptr(y, _u16p), M, H, _ptr(out["q"], _u8p),
                                            _ptr(out["scale"], _u8p))
        if rc != 0:
            raise ValueError("oracle rejected the arguments")
        return out

    # ---- the QK variant ----
    def qk_gemma_rmsnorm_gate(self, qg, k, q_w, k_w, Hq, Hk, D, eps) -> dict:
        qg, ld_qg = _rows(qg)
        k, ld_k = _rows(k)
        T = qg.shape[0]
        assert k.shape[0] == T
        q_w = np.ascontiguousarray(q_w, dtype=np.uint16)
        k_w = np.ascontiguousarray(k_w, dtype=np.uint16)
        out = dict(q=np.zeros((T, Hq, D), np.uint16), k=np.zeros((T, Hk, D), np.uint16),
                   gate=np.zeros((T, Hq, D), np.uint16))
        rc = self.lib.rq_ref_qk_gemma_rmsnorm_gate(
            _ptr(qg, _u16p), ld_qg, _ptr(k, _u16p), ld_k, _ptr(q_w, _u16p), _ptr(k_w, _u16p),
            T, Hq, Hk, D, eps, _ptr(out["q"], _u16p), _ptr(out["k"], _u16p),
            _ptr(out["gate"], _u16p))
        if rc != 0:
            raise ValueError("oracle rejected the arguments")
        return out

    def qk_gemma_rmsnorm_gate_fp8(self, qg, k, q_w, k_w, Hq, Hk, D, eps) -> dict:
        """The QK step with per-head FP8 outputs: q [T, Hq, D] and k [T, Hk, D]
        E4M3FN bytes, q_scale [T, Hq] and k_scale [T, Hk] fp32, gate bf16."""
        qg, ld_qg = _rows(qg)
        k, ld_k = _rows(k)
        T = qg.shape[0]
        assert k.shape[0] == T
        q_w = np.ascontiguousarray(q_w, dtype=np.uint16)
        k_w = np.ascontiguousarray(k_w, dtype=np.uint16)
        out = dict(q=np.zeros((T, Hq, D), np.uint8), q_scale=np.zeros((T, Hq), np.float32),
                   k=np.zeros((T, Hk, D), np.uint8), k_scale=np.zeros((T, Hk), np.float32),
                   gate=np.zeros((T, Hq, D), np.uint16))
        rc = self.lib.rq_ref_qk_gemma_rmsnorm_gate_fp8(
            _ptr(qg, _u16p), ld_qg, _ptr(k, _u16p), ld_k, _ptr(q_w, _u16p), _ptr(k_w, _u16p),
            T, Hq, Hk, D, eps, _ptr(out["q"], _u8p), _ptr(out["q_scale"], _f32p), _ptr(out["k"], _u8p),
            _ptr(out["k_scale"], _f32p), _ptr(out["gate"], _u16p))
        if rc != 0:
            raise ValueError("oracle rejected the arguments")
        return out

    def qk_gemma_rmsnorm_gate_mxfp4(self, qg, k, q_w, k_w, Hq, Hk, D, eps) -> dict:
        """The QK step with per-head MXFP4 outputs: q [T, Hq, D/2] and k [T, Hk, D/2]
        packed E2M1, q_scale [T, Hq, D/32] and k_scale [T, Hk, D/32] E8M0, gate bf16."""
        qg, ld_qg = _rows(qg)
        k, ld_k = _rows(k)
        T = qg.shape[0]
        assert k.shape[0] == T
        q_w = np.ascontiguousarray(q_w, dtype=np.uint16)
        k_w = np.ascontiguousarray(k_w, dtype=np.uint16)
        out = dict(q=np.zeros((T, Hq, D // 2), np.uint8), q_scale=np.zeros((T, Hq, D // 32), np.uint8),
                   k=np.zeros((T, Hk, D // 2), np.uint8), k_scale=np.zeros((T, Hk, D // 32), np.uint8),
                   gate=np.zeros((T, Hq, D), np.uint16))
        rc = self.lib.rq_ref_qk_gemma_rmsnorm_gate_mxfp4(
            _ptr(qg, _u16p), ld_qg, _ptr(k, _u16p), ld_k, _ptr(q_w, _u16p), _ptr(k_w, _u16p),
            T, Hq, Hk, D, eps, _ptr(out["q"], _u8p), _ptr(out["q_scale"], _u8p), _ptr(out["k"], _u8p),
            _ptr(out["k_scale"], _u8p), _ptr(out["gate"], _u16p))
        if rc != 0:
            raise ValueError("oracle rejected the arguments")
        return out


_DEFAULT: Oracle | None = None


def get() -> Oracle:
    """The process-wide oracle, building librq_oracle.so if it is missing."""
    global _DEFAULT
    if _DEFAULT is None:
        _DEFAULT = Oracle()
    return _DEFAULT
