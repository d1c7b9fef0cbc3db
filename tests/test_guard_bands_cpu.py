"""Negative controls of the guard-band checker of test_gpu_guard_bands.py, on
the CPU: a byte written before an output, after it, or into the padding
columns of a column-major scale array is reported; untouched buffers pass."""

import pytest
import torch

from test_gpu_guard_bands import GUARD, Guarded


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
