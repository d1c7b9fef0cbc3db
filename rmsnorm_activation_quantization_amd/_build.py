"""Build librmsnorm_quant.so in-tree with hipcc for gfx950."""

from __future__ import annotations

import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SOURCE = os.path.join(PKG, "csrc", "rmsnorm_quant.hip")
INCLUDE = os.path.join(ROOT, "include")
LIBRARY = os.path.join(PKG, "librmsnorm_quant.so")
# The same source with the per-launch grid limit lowered to 2^14 work-items, so
# that tests reach the multi-launch split of rows and QK heads with small
# batches (a test build only; nothing else loads it).
GRID_SPLIT_LIBRARY = os.path.join(PKG, "librmsnorm_quant_gridsplit.so")
GRID_SPLIT_FLAGS = ("-DRQ_MAX_GRID_ITEMS=16384",)
EXAMPLE_SOURCE = os.path.join(PKG, "csrc", "abi_example.c")
EXAMPLE = os.path.join(PKG, "rq_abi_example")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # every rounding is the one written in the source: no FMA contraction
    "-ffp-contract=off",
    # no packed fp32 instructions (v_pk_*_f32) anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def build(output: str = LIBRARY, extra_flags: tuple[str, ...] = ()) -> str:
    tmp = output + ".tmp"
    cmd = [HIPCC, *HIPCC_FLAGS, *extra_flags, "-I", INCLUDE, SOURCE, "-o", tmp]
    proc = subprocess.run(cmd, capture_output=True, text=True)
    if proc.returncode != 0:
        raise RuntimeError(f"hipcc failed ({proc.returncode}):\n{proc.stderr}")
    os.replace(tmp, output)
    return output


def build_example(output: str = EXAMPLE) -> str:
    """The plain-C user of the ABI (gcc, HIP runtime API only), linked against
    the library next to it."""
    cmd = ["gcc", "-std=c11", "-O2", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROCM, "include"), "-I", INCLUDE,
           EXAMPLE_SOURCE, "-o", output, "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-L", PKG,
           "-l:librmsnorm_quant.so", "-Wl,-rpath,$ORIGIN", "-Wl,-rpath," + os.path.join(ROCM, "lib")]
    proc = subprocess.run(cmd, capture_output=True, text=True)
    if proc.returncode != 0:
        raise RuntimeError(f"gcc failed ({proc.returncode}):\n{proc.stderr}")
    return output
