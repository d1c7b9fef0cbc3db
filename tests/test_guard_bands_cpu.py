"""The helpers of test_gpu_guard_bands.py, on the CPU: the guard-band checker
reports a byte written before an output, after it, or into the padding columns
of a column-major scale array, and passes untouched buffers; the NaN embedding
of inputs holds the values with NaN before, after and in every row's gap."""

import pytest
import torch

from test_gpu_guard_bands import GUARD, NAN_GAP, NAN_LEAD, Guarded, nan_embedded


def planted(where):
    g = Guarded("cpu")
    g.out((4, 8), torch.float32)
    s = g.out((3, 4), torch.uint8, ld=6)  # 3 scale rows of 4 columns, leading dimension 6
    base, nbytes = g.bufs[0][0], g.bufs[0][1]
    if where == "before":
        base[GUARD - 1] = 0
    elif where == "after":
        base[GUARD + nbytes] = 0
    elif where == "padding":
        s[2, 5] = 0
    return g


def test_untouched_buffers_pass():
    planted("nothing").check("untouched")


@pytest.mark.parametrize("where", ["before", "after", "padding"])
def test_writes_outside_outputs_are_reported(where):
    with pytest.raises(AssertionError, match="write"):
        planted(where).check(f"planted {where}")


def test_nan_embedding_surrounds_the_values():
    t = torch.arange(3 * 16, dtype=torch.float32).view(3, 16).to(torch.bfloat16)
    v = nan_embedded(t, device="cpu")
    assert torch.equal(v, t) and v.stride() == (16 + NAN_GAP, 1)
    flat = v.as_strided((NAN_LEAD + 3 * (16 + NAN_GAP) + NAN_LEAD,), (1,), v.storage_offset() - NAN_LEAD)
    mask = torch.ones_like(flat, dtype=torch.bool)
    for m in range(3):
        mask[NAN_LEAD + m * (16 + NAN_GAP):NAN_LEAD + m * (16 + NAN_GAP) + 16] = False
    assert torch.isnan(flat[mask]).all() and not torch.isnan(flat[~mask]).any()
    w = nan_embedded(torch.ones(8, dtype=torch.bfloat16), device="cpu")
    whole = w.as_strided((NAN_LEAD + 8 + NAN_LEAD,), (1,), w.storage_offset() - NAN_LEAD)
    assert torch.isnan(whole[:NAN_LEAD]).all() and torch.isnan(whole[NAN_LEAD + 8:]).all()
    assert torch.equal(whole[NAN_LEAD:NAN_LEAD + 8], torch.ones(8, dtype=torch.bfloat16))
