"""Host-side contract of bench.py (no GPU): the one-GPU refusal, and the
algorithmic bytes that `value` and `roofline` divide by."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


@pytest.mark.parametrize("argv,env", [(["--gpus", "2"], {}), (["--gpus", "8"], {}), ([], {"WORLD_SIZE": "4"})])
def test_more_than_one_gpu_is_refused(argv, env):
    """The path has no multi-GPU part: asked for several GPUs (by flag or by a
    launcher's WORLD_SIZE), bench.py says so and exits before touching a GPU."""
    proc = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *argv], capture_output=True, text=True,
                          env={**os.environ, **env}, timeout=120)
    assert proc.returncode == 2
    assert "one GPU only" in proc.stderr and proc.stdout == ""


def test_row_bytes():
    """Each tensor counted once: x, residual and residual_out (bf16), the
    weight, then codes and scales; the [8192, 4096] figures the roofline uses."""
    M, H = 8192, 4096
    rows = 2 * M * H * 3 + 2 * H
    assert bench.row_bytes("fp8_token", M, H) == rows + M * H + 4 * M == 234_921_984
    assert bench.row_bytes("fp8_group", M, H) == rows + M * H + 4 * M * (H // 128) == 235_937_792
    assert bench.row_bytes("fp8_group", M, H, group=32) == rows + M * H + 4 * M * (H // 32)
    assert bench.row_bytes("mxfp4", M, H) == rows + M * H // 2 + M * H // 32 == 219_160_576


def test_qk_bytes():
    """qg (q and gate interleaved) and k read, the two head weights read, q, k
    and gate written, all bf16: the decode call and 8192 tokens."""
    T, Hq, Hk, D = 64, 16, 2, 256
    reads = 2 * (T * 2 * Hq * D + T * Hk * D + 2 * D)
    writes = 2 * (T * Hq * D + T * Hk * D + T * Hq * D)
    assert bench.qk_bytes(T, Hq, Hk, D) == reads + writes == 2_229_248
    assert bench.qk_bytes(8192, Hq, Hk, D) == 285_213_696


def test_quantized_qk_bytes():
    """The quantized QK calls read what the bf16 one reads and write the bf16
    gate, with q and k as codes plus scales (FP8: a byte an element and one
    fp32 scale a head; MXFP4: half a byte an element and one byte per 32)."""
    T, Hq, Hk, D = 8192, 16, 2, 256
    reads = 2 * (T * 2 * Hq * D + T * Hk * D + 2 * D)
    gate = 2 * T * Hq * D
    heads = T * (Hq + Hk)
    assert bench.qk_fp8_bytes(T, Hq, Hk, D) == reads + gate + heads * D + 4 * heads == 248_054_784
    assert bench.qk_mxfp4_bytes(T, Hq, Hk, D) == reads + gate + heads * D // 2 + heads * D // 32 == 229_770_240
