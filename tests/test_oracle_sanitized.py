"""The oracle under sanitizers.

- Built with UndefinedBehaviorSanitizer checks in trap mode (g++
  -fsanitize=undefined,float-cast-overflow -fsanitize-undefined-trap-on-error:
  no runtime library; an undefined operation stops the process), with every
  pin run against that build in a process of its own.  Float division by zero
  is not trapped: the oracle's IEEE arithmetic relies on it (1/0 = inf).
- Built into an executable with AddressSanitizer and UndefinedBehaviorSanitizer
  beside oracle_asan_driver.cpp, which calls every entry point on heap buffers
  of exactly the extent its arguments describe.

Each has a negative control that the sanitizer must catch."""

import os
import subprocess
import sys
import textwrap

import oracle

TESTS = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(TESTS)
UB_FLAGS = ["-fsanitize=undefined,float-cast-overflow", "-fsanitize-undefined-trap-on-error"]


def pins_with_ub_trapped(source: str, lib: str) -> subprocess.CompletedProcess:
    """Builds `source` with the trap-mode checks into `lib` and runs the pins
    against it in a child process."""
    flags = [f for f in oracle.CXXFLAGS if not f.startswith("-O")] + ["-O1", "-g", *UB_FLAGS]
    build = subprocess.run(["g++", *flags, "-I", os.path.dirname(oracle.SOURCE), source, "-o", lib],
                           capture_output=True, text=True, timeout=600)
    assert build.returncode == 0, build.stderr[-4000:]
    script = textwrap.dedent(f"""
        import sys
        import pytest
        sys.path[:0] = [{ROOT!r}, {TESTS!r}]
        import oracle
        oracle._DEFAULT = oracle.Oracle({lib!r})
        assert oracle.get().lib._name == {lib!r}
        sys.exit(pytest.main(["-q", "-x", "-m", "not gpu", "-p", "no:cacheprovider",
                              {os.path.join(TESTS, "test_oracle_pins.py")!r}]))
    """)
    return subprocess.run([sys.executable, "-c", script], capture_output=True, text=True, timeout=900, cwd=ROOT)


def test_oracle_pins_pass_with_undefined_behaviour_trapped(tmp_path):
    run = pins_with_ub_trapped(oracle.SOURCE, str(tmp_path / "librq_oracle_ub.so"))
    assert run.returncode == 0, (run.returncode, run.stdout[-3000:], run.stderr[-3000:])
    assert " passed" in run.stdout


def test_planted_signed_overflow_is_trapped(tmp_path):
    """Negative control: the same run on a copy of the oracle whose bf16
    rounding first overflows a signed int stops at that operation."""
    src = open(oracle.SOURCE).read()
    head = "uint16_t bf16_round(double v) {"
    assert src.count(head) == 1
    planted = tmp_path / "rq_oracle_planted.cpp"
    planted.write_text(src.replace(head, head + " { volatile int big = 2147483647; big = big + 1; }"))
    run = pins_with_ub_trapped(str(planted), str(tmp_path / "librq_oracle_planted.so"))
    assert run.returncode == -4, (run.returncode, run.stdout[-2000:])  # SIGILL from the trap


def asan_driver(tmp_path, *args) -> subprocess.CompletedProcess:
    exe = str(tmp_path / "oracle_asan")
    flags = [f for f in oracle.CXXFLAGS if f not in ("-shared", "-fPIC") and not f.startswith("-O")]
    build = subprocess.run(["g++", *flags, "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                            "-I", os.path.dirname(oracle.SOURCE), os.path.join(TESTS, "oracle_asan_driver.cpp"),
                            oracle.SOURCE, "-o", exe], capture_output=True, text=True, timeout=600)
    assert build.returncode == 0, build.stderr[-4000:]
    return subprocess.run([exe, *args], capture_output=True, text=True, timeout=600)


def test_oracle_on_exact_buffers_under_asan(tmp_path):
    run = asan_driver(tmp_path, "300")
    assert run.returncode == 0 and "clean" in run.stdout, (run.returncode, run.stderr[-4000:])


def test_short_buffer_is_reported(tmp_path):
    """Negative control: the weight buffer one element short."""
    run = asan_driver(tmp_path, "300", "short")
    assert run.returncode != 0 and "heap-buffer-overflow" in run.stderr, (run.returncode, run.stderr[-2000:])
