"""Negative controls of the parity checker (tests/parity.py), on the CPU.

Every GPU parity test is judged by check_fp8, check_mxfp4 and check_bf16_close.
Here each is fed the oracle's own outputs standing in for the GPU's, first
unmodified (they must pass), then with one planted difference each (it must be
rejected).  A planted code, scale or E8M0 difference is planted twice: once in
the stand-in GPU outputs alone (the exact re-quantization check must catch it),
and once in both the stand-in outputs and their re-quantization (so that the
exact check passes and the tolerance checks against the oracle's full result
must catch it on their own).
"""

from __future__ import annotations

import numpy as np
import pytest

from parity import CODE_MATCH_MIN, Y_FLIP_RATE_MAX, check_bf16_close, check_fp8, check_mxfp4, code_steps
from rmsnorm_activation_quantization_amd import inputs

M, H = 32, 512
EPS = 1e-6


def _rows(seed=4242, zero_frac=0.02):
    """Seeded rows in which a fraction of elements cancel exactly (x = -residual),
    so that r, y and the codes there are +0: material for sign-of-zero controls."""
    d = inputs.random_rows(M, H, seed)
    xb, rb, wb = (inputs.bits(d[k]) for k in ("x", "residual", "weight"))
    rng = np.random.default_rng(seed)
    z = rng.random((M, H)) < zero_frac
    rb = np.where(z, xb ^ 0x8000, rb).astype(np.uint16)
    return xb, rb, wb


def _fp8_case(ref, granule):
    xb, rb, wb = _rows()
    if granule == H:
        o = ref.fp8_per_token(xb, rb, wb, EPS, emit_y=True)
        o["scale"] = o["scale"].reshape(M, 1)
    else:
        o = ref.fp8_per_group(xb, rb, wb, EPS, granule, emit_y=True)
    gpu = {k: v.copy() for k, v in o.items()}
    requant = ref.quantize_fp8(gpu["y"], granule)
    requant["scale"] = requant["scale"].reshape(gpu["scale"].shape)
    return gpu, o, requant


def _mx_case(ref):
    xb, rb, wb = _rows()
    o = ref.mxfp4(xb, rb, wb, EPS, emit_y=True)
    gpu = {k: v.copy() for k, v in o.items()}
    return gpu, o, ref.quantize_mxfp4(gpu["y"])


def _pick(mask):
    idx = np.argwhere(mask)
    assert len(idx), "no element fits the planted difference"
    return tuple(idx[len(idx) // 2])


def _count_for_rate(n, rate):
    """Elements to plant so that a rate-based check is exceeded."""
    return int(np.ceil(n * rate)) + 2


# ---- the unmodified outputs pass ----

@pytest.mark.parametrize("granule", [H, 128])
def test_fp8_unmodified_passes(ref, granule):
    gpu, o, rq = _fp8_case(ref, granule)
    stats = check_fp8(gpu, o, rq, granule, "unmodified")
    assert stats["flips"] == 0 and stats["code_match"] == 1.0 and stats["scale_diffs"] == 0


def test_mxfp4_unmodified_passes(ref):
    gpu, o, rq = _mx_case(ref)
    stats = check_mxfp4(gpu, o, rq, "unmodified")
    assert stats["flips"] == 0 and stats["code_match"] == 1.0 and stats["scale_diffs"] == 0


def test_rows_hold_zero_codes(ref):
    """The fixture rows really contain +0 codes, so the sign-of-zero controls bite."""
    gpu, _, _ = _fp8_case(ref, 128)
    assert (gpu["q"] == 0x00).mean() > 0.01
    gm, _, _ = _mx_case(ref)
    assert ((gm["q"] & 0xF) == 0).mean() > 0.01


# ---- bf16 rows ----

def test_bf16_two_ulps_rejected(ref):
    gpu, o, _ = _fp8_case(ref, H)
    y = gpu["y"].copy()
    i = _pick((y & 0x7FFF) > 0x100)
    y[i] += 2
    with pytest.raises(AssertionError, match="bf16 ulps apart"):
        check_bf16_close(y, o["y"], "planted")


def test_bf16_flip_rate_rejected(ref):
    gpu, o, _ = _fp8_case(ref, H)
    y = gpu["y"].copy().reshape(-1)
    n = _count_for_rate(y.size, Y_FLIP_RATE_MAX)
    idx = np.flatnonzero((y & 0x7FFF) > 0x100)[:n]
    y[idx] += 1
    with pytest.raises(AssertionError, match="flipped by one ulp"):
        check_bf16_close(y, o["y"].reshape(-1), "planted")
    # the same count below the rate is accepted, and counted
    y2 = o["y"].copy().reshape(-1)
    y2[idx[:3]] += 1
    assert check_bf16_close(y2, o["y"].reshape(-1), "three flips")["flips"] == 3


def test_bf16_zero_sign_counts_as_a_flip(ref):
    gpu, o, _ = _fp8_case(ref, H)
    y = gpu["y"].copy().reshape(-1)
    zeros = np.flatnonzero(y == 0x0000)
    y[zeros[0]] = 0x8000
    assert check_bf16_close(y, o["y"].reshape(-1), "one -0")["flips"] == 1
    y[zeros[: _count_for_rate(y.size, Y_FLIP_RATE_MAX)]] = 0x8000
    with pytest.raises(AssertionError, match="flipped by one ulp"):
        check_bf16_close(y, o["y"].reshape(-1), "many -0")


def test_code_steps_line():
    """+0 and -0 one step apart; the smallest magnitudes of either sign two apart."""
    assert code_steps(np.array([0x00]), np.array([0x80]), 0x80)[0] == 1
    assert code_steps(np.array([0x01]), np.array([0x81]), 0x80)[0] == 2
    assert code_steps(np.array([0x01]), np.array([0x00]), 0x80)[0] == 1
    assert code_steps(np.array([0x8]), np.array([0x0]), 0x8)[0] == 1
    assert code_steps(np.array([0x7E]), np.array([0x7C]), 0x80)[0] == 2


# ---- FP8 ----

@pytest.mark.parametrize("granule", [H, 128])
def test_fp8_residual_bit_rejected(ref, granule):
    gpu, o, rq = _fp8_case(ref, granule)
    gpu["residual_out"][3, 7] ^= 1
    with pytest.raises(AssertionError, match="residual_out"):
        check_fp8(gpu, o, rq, granule, "planted")


@pytest.mark.parametrize("granule", [H, 128])
def test_fp8_y_two_ulps_rejected(ref, granule):
    gpu, o, rq = _fp8_case(ref, granule)
    gpu["y"][_pick((gpu["y"] & 0x7FFF) > 0x100)] += 2
    with pytest.raises(AssertionError, match="bf16 ulps apart"):
        check_fp8(gpu, o, rq, granule, "planted")


@pytest.mark.parametrize("granule", [H, 128])
@pytest.mark.parametrize("also_requant", [False, True])
def test_fp8_code_two_steps_rejected(ref, granule, also_requant):
    gpu, o, rq = _fp8_case(ref, granule)
    i = _pick(((gpu["q"] & 0x7F) > 4) & ((gpu["q"] & 0x7F) < 0x70))
    gpu["q"][i] += 2
    if also_requant:
        rq["q"][i] += 2
    with pytest.raises(AssertionError, match="quantize\\(y_gpu\\)" if not also_requant else "steps from the oracle"):
        check_fp8(gpu, o, rq, granule, "planted")


@pytest.mark.parametrize("granule", [H, 128])
def test_fp8_one_step_codes_beyond_match_rate_rejected(ref, granule):
    gpu, o, rq = _fp8_case(ref, granule)
    flat = np.flatnonzero(((gpu["q"] & 0x7F) > 4) & ((gpu["q"] & 0x7F) < 0x70))
    idx = np.unravel_index(flat[: _count_for_rate(gpu["q"].size, 1 - CODE_MATCH_MIN)], gpu["q"].shape)
    gpu["q"][idx] += 1
    rq["q"][idx] += 1
    with pytest.raises(AssertionError, match="of codes identical"):
        check_fp8(gpu, o, rq, granule, "planted")


@pytest.mark.parametrize("granule", [H, 128])
@pytest.mark.parametrize("also_requant", [False, True])
def test_fp8_scale_moved_rejected(ref, granule, also_requant):
    """A scale one fp32 ulp off, with the granule's amax unchanged."""
    gpu, o, rq = _fp8_case(ref, granule)
    gpu["scale"].view(np.uint32)[1, 0] += 1
    if also_requant:
        rq["scale"].view(np.uint32)[1, 0] += 1
    with pytest.raises(AssertionError, match="scales differ" if not also_requant else "one-ulp amax change"):
        check_fp8(gpu, o, rq, granule, "planted")


@pytest.mark.parametrize("granule", [H, 128])
def test_fp8_zero_sign_beyond_match_rate_rejected(ref, granule):
    gpu, o, rq = _fp8_case(ref, granule)
    zeros = np.flatnonzero(gpu["q"] == 0x00)
    n = _count_for_rate(gpu["q"].size, 1 - CODE_MATCH_MIN)
    assert len(zeros) >= n
    idx = np.unravel_index(zeros[:n], gpu["q"].shape)
    gpu["q"][idx] = 0x80
    rq["q"][idx] = 0x80
    with pytest.raises(AssertionError, match="of codes identical"):
        check_fp8(gpu, o, rq, granule, "planted")


def test_fp8_wrong_granule_rejected(ref):
    """Per-group outputs judged as if their scales were one per token: the
    shapes disagree, so the check cannot pass by accident."""
    gpu, o, rq = _fp8_case(ref, 128)
    with pytest.raises((AssertionError, ValueError)):
        check_fp8(gpu, o, rq, H, "planted")


# ---- MXFP4 ----

def test_mxfp4_residual_bit_rejected(ref):
    gpu, o, rq = _mx_case(ref)
    gpu["residual_out"][5, 9] ^= 0x10
    with pytest.raises(AssertionError, match="residual_out"):
        check_mxfp4(gpu, o, rq, "planted")


def test_mxfp4_swapped_nibbles_rejected(ref):
    gpu, o, rq = _mx_case(ref)
    q = gpu["q"]
    i = _pick((q & 0xF) != (q >> 4))
    q[i] = ((q[i] & 0xF) << 4) | (q[i] >> 4)
    with pytest.raises(AssertionError, match="quantize\\(y_gpu\\)"):
        check_mxfp4(gpu, o, rq, "planted")


def test_mxfp4_all_nibbles_swapped_rejected(ref):
    """Low and high nibble exchanged in every byte, in the outputs and their
    re-quantization alike (an element order mistake on both sides)."""
    gpu, o, rq = _mx_case(ref)
    for d in (gpu, rq):
        d["q"] = (((d["q"] & 0xF) << 4) | (d["q"] >> 4)).astype(np.uint8)
    with pytest.raises(AssertionError, match="of codes identical"):
        check_mxfp4(gpu, o, rq, "planted")


@pytest.mark.parametrize("also_requant", [False, True])
def test_mxfp4_code_two_steps_rejected(ref, also_requant):
    gpu, o, rq = _mx_case(ref)
    q = gpu["q"]
    i = _pick(((q & 0x7) >= 1) & ((q & 0x7) <= 5))
    q[i] += 2  # low nibble two codes up, inside its sign
    if also_requant:
        rq["q"][i] += 2
    with pytest.raises(AssertionError, match="quantize\\(y_gpu\\)" if not also_requant else "steps from the oracle"):
        check_mxfp4(gpu, o, rq, "planted")


@pytest.mark.parametrize("also_requant", [False, True])
def test_mxfp4_e8m0_off_by_two_rejected(ref, also_requant):
    gpu, o, rq = _mx_case(ref)
    gpu["scale"][2, 3] += 2
    if also_requant:
        rq["scale"][2, 3] += 2
    with pytest.raises(AssertionError, match="E8M0"):
        check_mxfp4(gpu, o, rq, "planted")


def test_mxfp4_zero_sign_beyond_match_rate_rejected(ref):
    gpu, o, rq = _mx_case(ref)
    lo_zero = np.flatnonzero((gpu["q"] & 0xF) == 0)
    n = _count_for_rate(2 * gpu["q"].size, 1 - CODE_MATCH_MIN)
    assert len(lo_zero) >= n
    idx = np.unravel_index(lo_zero[:n], gpu["q"].shape)
    gpu["q"][idx] |= 0x8
    rq["q"][idx] |= 0x8
    with pytest.raises(AssertionError, match="of codes identical"):
        check_mxfp4(gpu, o, rq, "planted")


def test_mxfp4_e8m0_off_by_one_without_amax_change_rejected(ref):
    """An E8M0 byte one off where the block's amax did not move (planted in the
    outputs and their re-quantization alike): only a one-ulp amax change
    across a power of two may move it."""
    gpu, o, rq = _mx_case(ref)
    gpu["scale"][4, 1] += 1
    rq["scale"][4, 1] += 1
    with pytest.raises(AssertionError, match="without a one-ulp amax change"):
        check_mxfp4(gpu, o, rq, "planted")


# ---- MXFP4 blocks whose E8M0 byte legitimately moved ----

def _probe_block(ref):
    """20 equal rows, H = 2048, through the oracle with x = residual = 512 and eps = 0, so
    that y equals the weight bit for bit.  Block 0 holds amax 4.0 (E8M0 127)
    and 2.875 (code 3.0 at scale 1, index 5).  The stand-in GPU row has the
    4.0 one ulp lower (3.984375): its block byte is 126, and 2.875 encodes as
    6.0 at scale 1/2 (index 7), the same value two indices away."""
    from parity import mxfp4_value_steps  # noqa: F401  (imported where it is used below)
    H = 2048
    w = np.full(H, 0x3F80, np.uint16)          # 1.0
    w[0], w[1] = 0x4080, 0x4038                # 4.0, 2.875
    xb = np.full((20, H), 0x4400, np.uint16)  # 512
    o = ref.mxfp4(xb, xb, w, 0.0, emit_y=True)
    assert (o["y"] == w).all() and o["scale"][0, 0] == 127
    gy = o["y"].copy()
    gy[0, 0] = 0x407F                          # 3.984375, one ulp below 4.0
    rq = ref.quantize_mxfp4(gy)
    gpu = dict(residual_out=o["residual_out"].copy(), y=gy, q=rq["q"].copy(), scale=rq["scale"].copy())
    assert gpu["scale"][0, 0] == 126
    return gpu, o, rq


def test_mxfp4_moved_byte_same_value_accepted(ref):
    gpu, o, rq = _probe_block(ref)
    # element 1: oracle index 5 (3.0 under 2^0), stand-in index 7 (6.0 under 2^-1)
    assert (o["q"][0, 0] >> 4) == 5 and (gpu["q"][0, 0] >> 4) == 7
    stats = check_mxfp4(gpu, o, rq, "moved byte")
    assert stats["scale_diffs"] == 1


def test_mxfp4_moved_byte_value_two_coarse_steps_rejected(ref):
    gpu, o, rq = _probe_block(ref)
    for d in (gpu, rq):
        d["q"][0, 0] = (d["q"][0, 0] & 0x0F) | (5 << 4)   # 3.0 under 2^-1 = 1.5 against the oracle's 3.0
    with pytest.raises(AssertionError, match="coarser grid"):
        check_mxfp4(gpu, o, rq, "planted")


def test_mxfp4_value_steps():
    from parity import mxfp4_value_steps
    one = np.array([1])
    # equal bytes: adjacent codes one step, 1.5 -> 3 two steps (spacing 1 above 2)
    assert mxfp4_value_steps(np.array([3]), 127 * one, np.array([4]), 127 * one)[0] == 1.0
    assert mxfp4_value_steps(np.array([3]), 127 * one, np.array([5]), 127 * one)[0] == 1.5
    assert mxfp4_value_steps(np.array([6]), 127 * one, np.array([7]), 127 * one)[0] == 1.0
    # bytes one apart: 6.0 under 2^-1 equals 3.0 under 2^0
    assert mxfp4_value_steps(np.array([7]), 126 * one, np.array([5]), 127 * one)[0] == 0.0
    # signs: -0.5 and +0.5 are two steps apart
    assert mxfp4_value_steps(np.array([0x9]), 127 * one, np.array([0x1]), 127 * one)[0] == 2.0
