"""The C++ reference loops under AddressSanitizer and UndefinedBehaviorSanitizer.

oracle/moe_oracle_ref.cpp is compiled with g++ together with the driver
tests/oracle_sanitize_main.cpp (every entry point on tiny and degenerate
inputs, invariant checks) into a stand-alone program, run as a child process
so that the sanitizer runtimes never load into the Python interpreter.  Any
out-of-bounds access, use after free, leak, null argument to a library
routine or other undefined behaviour ends the run with a report.  A second
build plants a caller-side overflow (an offsets array one element short) to
show that the sanitizers are really active in this toolchain."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SOURCES = [os.path.join(ROOT, "oracle", "moe_oracle_ref.cpp"), os.path.join(ROOT, "tests", "oracle_sanitize_main.cpp")]
FLAGS = ["-O1", "-g", "-fno-omit-frame-pointer", "-fopenmp", "-fsanitize=address,undefined",
         "-fno-sanitize-recover=all"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:exitcode=23",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", OMP_NUM_THREADS="2")


def _build(tmp, name, extra=()):
    if shutil.which("g++") is None:
        pytest.skip("g++ is not installed")
    exe = os.path.join(tmp, name)
    r = subprocess.run(["g++", *FLAGS, *extra, *SOURCES, "-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    return exe


@pytest.fixture(scope="module")
def tmpdir_mod(tmp_path_factory):
    return str(tmp_path_factory.mktemp("oracle_san"))


def test_oracle_clean_under_asan_ubsan(tmpdir_mod):
    exe = _build(tmpdir_mod, "oracle_san")
    r = subprocess.run([exe], capture_output=True, text=True, env=ENV, timeout=300)
    report = r.stdout + r.stderr
    assert r.returncode == 0, report[-6000:]
    assert "runtime error" not in report and "AddressSanitizer" not in report, report[-6000:]
    assert "all checks held" in r.stdout


def test_sanitizer_catches_planted_overflow(tmpdir_mod):
    exe = _build(tmpdir_mod, "oracle_san_planted", ["-DPLANT_SHORT_OFFSETS"])
    r = subprocess.run([exe], capture_output=True, text=True, env=ENV, timeout=300)
    assert r.returncode != 0
    assert "heap-buffer-overflow" in r.stderr
    assert "oracle_permute" in r.stderr
