"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module holds only random-number recipes: no part of the method's
arithmetic.  Every tensor is drawn in fp32 on torch's CPU generator and rounded
once (nearest-even) to bf16.  The pages measure on trained checkpoints and
serving workloads that are not available here; these rows of the same shapes
stand in for them.

Recipes (one seed per workload, draws in the fixed order x, residual, weight,
then the outlier masks):
  x, residual ~ N(0, 1); weight ~ N(1, 0.1)
  "outliers": every element of x and, independently, of residual is
              multiplied by 20 with probability 0.01 (before the bf16 rounding)
  QK: qg, k ~ N(0, 1); q_w, k_w ~ N(0, 0.1) (applied as 1 + w by the method)
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch


@dataclass(frozen=True)
class RowWorkload:
    name: str
    M: int
    H: int
    seed: int
    outliers: bool = False
    eps: float = 1e-6


@dataclass(frozen=True)
class QKWorkload:
    name: str
    T: int
    Hq: int
    Hk: int
    D: int
    seed: int
    eps: float = 1e-6


# The five workloads of the method's statement.
FP8_TOKEN_SMALL = RowWorkload("fp8_per_token_4x2048", 4, 2048, 1001)
FP8_GROUP_DECODE = RowWorkload("fp8_per_group128_16x4096_outliers", 16, 4096, 1002, outliers=True)
MXFP4_DECODE = RowWorkload("mxfp4_16x7168", 16, 7168, 1003)
QK_DECODE = QKWorkload("qk_gemma_gate_64x16x2x256", 64, 16, 2, 256, 1004)
PREFILL = RowWorkload("prefill_8192x4096", 8192, 4096, 1005)
# The decode size the headline metric is quoted at (all three formats).
DECODE_4096 = RowWorkload("decode_16x4096", 16, 4096, 1006)


def _normal(gen: torch.Generator, shape, mean: float, std: float) -> torch.Tensor:
    return torch.randn(shape, generator=gen, dtype=torch.float32) * std + mean


def row_inputs(w: RowWorkload, set_index: int = 0, dtype: torch.dtype = torch.bfloat16) -> dict:
    """x, residual [M, H] and weight [H] as CPU tensors of `dtype` (bf16 or fp16;
    the same fp32 draws, rounded once to that type)."""
    gen = torch.Generator().manual_seed(w.seed + 7919 * set_index)
    x = _normal(gen, (w.M, w.H), 0.0, 1.0)
    residual = _normal(gen, (w.M, w.H), 0.0, 1.0)
    weight = _normal(gen, (w.H,), 1.0, 0.1)
    if w.outliers:
        x = torch.where(torch.rand((w.M, w.H), generator=gen) < 0.01, x * 20.0, x)
        residual = torch.where(torch.rand((w.M, w.H), generator=gen) < 0.01, residual * 20.0, residual)
    return dict(x=x.to(dtype), residual=residual.to(dtype), weight=weight.to(dtype))


def qk_inputs(w: QKWorkload, ld_k: int | None = None) -> dict:
    """qg [T, 2*Hq*D], k [T, ld_k] (the first Hk*D columns are the heads),
    q_w, k_w [D], as CPU bf16 tensors."""
    gen = torch.Generator().manual_seed(w.seed)
    qg = _normal(gen, (w.T, 2 * w.Hq * w.D), 0.0, 1.0)
    k = _normal(gen, (w.T, ld_k or w.Hk * w.D), 0.0, 1.0)
    q_w = _normal(gen, (w.D,), 0.0, 0.1)
    k_w = _normal(gen, (w.D,), 0.0, 0.1)
    return dict(qg=qg.to(torch.bfloat16), k=k.to(torch.bfloat16),
                q_w=q_w.to(torch.bfloat16), k_w=k_w.to(torch.bfloat16))


def random_rows(M: int, H: int, seed: int, dtype: torch.dtype = torch.bfloat16) -> dict:
    """Generic seeded rows for edge-case shapes (same distributions)."""
    return row_inputs(RowWorkload(f"rows_{M}x{H}", M, H, seed), 0, dtype)


def bits(t: torch.Tensor) -> np.ndarray:
    """The uint16 bit patterns of a bf16 or fp16 tensor (any device), as numpy."""
    assert t.dtype in (torch.bfloat16, torch.float16)
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def from_bits(a: np.ndarray, dtype: torch.dtype = torch.bfloat16) -> torch.Tensor:
    """A CPU bf16 (or fp16) tensor from uint16 bit patterns."""
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint16).view(np.int16)).view(dtype)
