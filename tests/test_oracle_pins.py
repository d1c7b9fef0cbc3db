"""The CPU oracle against its pins (formats, hand-derived goldens, closed
forms, an independent numpy formulation, invariants).  No GPU needed."""

import numpy as np
import pytest

from oracle_pins import ALL_PINS, every_e8m0_byte_blocks, np_mxfp4


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(ref, pin):
    pin(ref)


@pytest.mark.parametrize("dtype,n_bytes", [("bf16", 253), ("fp16", 40)])
def test_oracle_mxfp4_every_scale_byte(ref, dtype, n_bytes):
    """The oracle's MXFP4 quantization against the independent numpy one (nearest
    value on the E2M1 grid after an frexp-derived scale) on blocks that put
    every magnitude of the type under every E8M0 byte it can sit under.  Kept
    out of the pin list the negative controls rerun, for its size (8.6 M bf16
    elements)."""
    bits = every_e8m0_byte_blocks(dtype)
    o = ref.quantize_mxfp4(bits, dtype=dtype)
    q, byte = np_mxfp4(bits, dtype)
    assert len(np.unique(byte)) == n_bytes
    assert (o["scale"] == byte).all(), "E8M0 bytes differ from the numpy formulation"
    assert (o["q"] == q).all(), "E2M1 codes differ from the numpy formulation"
