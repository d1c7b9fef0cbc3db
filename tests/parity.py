"""Comparison of the HIP path against the oracle (used by the GPU tests).

Tolerances (the method statement's, written here):
  residual_out              bit-exact (a correctly rounded bf16 sum on both sides)
  y (bf16 normalized row)   within 1 bf16 ulp; the flip rate is reported.  The
                            kernel computes rstd in fp32, the oracle in fp64, so
                            y can differ where r * rstd * w lies next to a bf16
                            rounding boundary.
  codes                     identical on >= 99.9 % of elements, the rest at most
                            one code step apart;
  scales                    equal, or moved only where the granule's amax
                            moved by exactly one bf16 ulp (FP8: the scale of
                            amax +- 1 ulp; E8M0: +- 1 where that crosses a
                            power of two).
  Stronger, exact check: the kernel's codes and scales are bit-identical to the
  oracle's quantization of the kernel's own y (the quantizer is a pure function
  of the bf16 row, so nothing excuses a difference there).
QK: q and k within 1 bf16 ulp, gate bit-exact.
"""

from __future__ import annotations

import numpy as np

from rmsnorm_activation_quantization_amd import inputs

Y_FLIP_RATE_MAX = 1e-3
CODE_MATCH_MIN = 0.999


def signed_key(bits: np.ndarray, sign_bit: int) -> np.ndarray:
    """Sign-magnitude codes mapped onto a monotonic integer line (+0 and -0 both 0)."""
    b = np.asarray(bits).astype(np.int64)
    mag = b & (sign_bit - 1)
    return np.where(b & sign_bit, -mag, mag)


def code_steps(a, b, sign_bit: int) -> np.ndarray:
    """Steps between sign-magnitude codes along the line of representable values,
    with +0 and -0 one step apart.  Both sides keep the sign of zero (a zero
    carries the sign of the product that rounded to it), so a zero of the
    wrong sign counts as a one-step difference rather than as a match."""
    a, b = np.asarray(a).astype(np.int64), np.asarray(b).astype(np.int64)
    mask = sign_bit - 1
    zero_sign = ((a & mask) == 0) & ((b & mask) == 0) & (a != b)
    return np.abs(signed_key(a, sign_bit) - signed_key(b, sign_bit)) + zero_sign


def bf16_ulps(a, b) -> np.ndarray:
    return code_steps(a, b, 0x8000)


E2M1_MAGNITUDES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def mxfp4_value_steps(g, g_byte, r, r_byte) -> np.ndarray:
    """Distance between E2M1 codes g and r (nibbles) held under E8M0 bytes g_byte
    and r_byte (broadcast to the codes), in steps of the E2M1 grid of the coarser
    scale around the larger magnitude (0.5 up to 2, 1 up to 4, 2 above).  Where
    the bytes are equal and the codes adjacent this is one step; where a block's
    byte moved by one, codes whose values agree (3.0 under 2^e, 6.0 under
    2^(e-1)) are zero steps apart although their indices differ by two."""
    g, r = np.asarray(g).astype(np.int64), np.asarray(r).astype(np.int64)
    e = np.maximum(g_byte, r_byte).astype(np.int64)
    vg = np.where(g & 8, -1.0, 1.0) * E2M1_MAGNITUDES[g & 7] * np.exp2(np.asarray(g_byte, np.int64) - e)
    vr = np.where(r & 8, -1.0, 1.0) * E2M1_MAGNITUDES[r & 7] * np.exp2(np.asarray(r_byte, np.int64) - e)
    m = np.maximum(np.abs(vg), np.abs(vr))
    spacing = np.where(m <= 2.0, 0.5, np.where(m <= 4.0, 1.0, 2.0))
    return np.abs(vg - vr) / spacing


def check_bf16_close(got, want, what: str, max_flip_rate: float = Y_FLIP_RATE_MAX) -> dict:
    d = bf16_ulps(got, want)
    assert d.max(initial=0) <= 1, f"{what}: {int(d.max())} bf16 ulps apart at {np.argwhere(d > 1)[:5].tolist()}"
    rate = float((d != 0).mean()) if d.size else 0.0
    assert rate <= max_flip_rate, f"{what}: {rate:.2e} of values flipped by one ulp"
    return {"flips": int((d != 0).sum()), "flip_rate": rate}


def to_np(out: dict) -> dict:
    import torch
    res = {}
    for k, v in out.items():
        if v is None:
            res[k] = None
        elif v.dtype in (torch.bfloat16, torch.float16):
            res[k] = inputs.bits(v)
        elif v.dtype == torch.float8_e4m3fn:
            res[k] = v.view(torch.uint8).cpu().numpy()
        else:
            res[k] = v.cpu().numpy()
    return res


def check_fp8(gpu: dict, ref: dict, requant: dict, granule: int, what: str) -> dict:
    """gpu/ref: residual_out, y, q [M,H] uint8, scale [M,G] fp32; requant: oracle quantize(gpu y)."""
    M, H = gpu["q"].shape
    assert (gpu["residual_out"] == ref["residual_out"]).all(), f"{what}: residual_out not bit-exact"
    stats = check_bf16_close(gpu["y"], ref["y"], f"{what}: y")
    # exact: the kernel quantized its own y exactly as the oracle would
    assert (gpu["q"] == requant["q"]).all(), f"{what}: codes differ from quantize(y_gpu)"
    assert np.array_equal(gpu["scale"].view(np.uint32), requant["scale"].reshape(gpu["scale"].shape).view(np.uint32)), \
        f"{what}: scales differ from quantize(y_gpu)"
    # tolerance against the oracle's full result
    same = gpu["q"] == ref["q"]
    match = float(same.mean())
    assert match >= CODE_MATCH_MIN, f"{what}: only {match:.5f} of codes identical"
    nan = ((ref["q"] & 0x7F) == 0x7F) | ((gpu["q"] & 0x7F) == 0x7F)
    steps = code_steps(gpu["q"], ref["q"], 0x80)[~nan]
    assert steps.max(initial=0) <= 1, f"{what}: a code is {int(steps.max())} steps from the oracle's"
    gs = gpu["scale"].reshape(M, H // granule)
    rs = ref["scale"].reshape(M, H // granule)
    diff = gs.view(np.uint32) != rs.view(np.uint32)
    if diff.any():
        ya = (gpu["y"].astype(np.int64) & 0x7FFF).reshape(M, H // granule, granule).max(axis=2)
        yr = (ref["y"].astype(np.int64) & 0x7FFF).reshape(M, H // granule, granule).max(axis=2)
        assert (np.abs(ya - yr)[diff] == 1).all(), f"{what}: a scale differs without a one-ulp amax change"
    stats.update(code_match=match, scale_diffs=int(diff.sum()))
    return stats


def check_mxfp4(gpu: dict, ref: dict, requant: dict, what: str) -> dict:
    M = gpu["q"].shape[0]
    assert (gpu["residual_out"] == ref["residual_out"]).all(), f"{what}: residual_out not bit-exact"
    stats = check_bf16_close(gpu["y"], ref["y"], f"{what}: y")
    assert (gpu["q"] == requant["q"]).all(), f"{what}: codes differ from quantize(y_gpu)"
    assert (gpu["scale"] == requant["scale"]).all(), f"{what}: E8M0 bytes differ from quantize(y_gpu)"
    nib = lambda q: np.stack([q & 0xF, q >> 4], axis=-1).reshape(M, -1)
    g, r = nib(gpu["q"]), nib(ref["q"])
    match = float((g == r).mean())
    assert match >= CODE_MATCH_MIN, f"{what}: only {match:.5f} of codes identical"
    bd = np.abs(gpu["scale"].astype(int) - ref["scale"].astype(int))
    assert bd.max(initial=0) <= 1, f"{what}: an E8M0 byte differs by {int(bd.max())}"
    if bd.any():
        nb = gpu["y"].shape[1] // 32
        ya = (gpu["y"].astype(np.int64) & 0x7FFF).reshape(M, nb, 32).max(axis=2)
        yr = (ref["y"].astype(np.int64) & 0x7FFF).reshape(M, nb, 32).max(axis=2)
        assert (np.abs(ya - yr)[bd != 0] == 1).all(), f"{what}: an E8M0 byte differs without a one-ulp amax change"
    # Codes under equal E8M0 bytes: at most one step apart on the code line.
    # Under bytes one apart (the one-ulp amax change across a power of two just
    # checked) the codes sit on grids a factor of two apart: compare their
    # values, at most one step of the coarser grid.
    same = np.repeat(bd == 0, 32, axis=1)
    steps = code_steps(g, r, 0x8)[same]
    assert steps.max(initial=0) <= 1, f"{what}: a code is {int(steps.max())} steps from the oracle's"
    if (~same).any():
        gb = np.repeat(gpu["scale"].astype(np.int64), 32, axis=1)
        rb = np.repeat(ref["scale"].astype(np.int64), 32, axis=1)
        vs = mxfp4_value_steps(g[~same], gb[~same], r[~same], rb[~same])
        assert vs.max(initial=0) <= 1, f"{what}: a code is {vs.max():.2f} steps of the coarser grid from the oracle's"
    stats.update(code_match=match, scale_diffs=int((bd != 0).sum()))
    return stats
