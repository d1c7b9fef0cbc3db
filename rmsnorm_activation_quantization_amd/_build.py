"""Build librmsnorm_quant.so in-tree with hipcc for gfx950."""

from __future__ import annotations

import os
import subprocess
import sysconfig

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


MARSHAL_SOURCE = os.path.join(PKG, "csrc", "marshal.cpp")


def marshal_path() -> str:
    """The CPython module of the binding's argument marshalling, in-tree."""
    return os.path.join(PKG, "_marshal" + sysconfig.get_config_var("EXT_SUFFIX"))


def build_marshal(output: str | None = None) -> str:
    """The binding's marshalling module (host C++ against torch's headers, g++;
    no device code)."""
    import torch.utils.cpp_extension as ce

    output = output or marshal_path()
    torch_lib = ce.library_paths()[0]
    cmd = ["g++", "-O2", "-std=c++17", "-fPIC", "-shared", "-D__HIP_PLATFORM_AMD__=1", "-DUSE_ROCM=1",
           f"-D_GLIBCXX_USE_CXX11_ABI={int(__import__('torch')._C._GLIBCXX_USE_CXX11_ABI)}",
           *[f"-I{p}" for p in ce.include_paths()], "-I", os.path.join(ROCM, "include"),
           "-I", sysconfig.get_paths()["include"], MARSHAL_SOURCE, "-o", output + ".tmp",
           f"-L{torch_lib}", "-ltorch", "-ltorch_cpu", "-lc10", "-lc10_hip", "-ltorch_python", f"-Wl,-rpath,{torch_lib}"]
    proc = subprocess.run(cmd, capture_output=True, text=True)
    if proc.returncode != 0:
        raise RuntimeError(f"g++ failed ({proc.returncode}):\n{proc.stderr}")
    os.replace(output + ".tmp", output)
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
