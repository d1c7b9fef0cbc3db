"""The C ABI driven from plain C (csrc/abi_example.c): HIP runtime allocation
and a stream, the fused, unfused and QK entry points, closed-form results and
the preflight errors, with no Python or torch in the process."""

import os
import subprocess

import pytest

from rmsnorm_activation_quantization_amd import _build

pytestmark = pytest.mark.gpu


def test_plain_c_program():
    assert os.path.exists(_build.EXAMPLE), "build the package first (it also builds the C example)"
    out = subprocess.run([_build.EXAMPLE], capture_output=True, text=True, timeout=120)
    assert out.returncode == 0 and "abi example ok" in out.stdout, out.stdout + out.stderr
