"""The C ABI's host code under AddressSanitizer and UBSan.

A second build of the library instruments kda_abi.cpp's host code (argument
validation, workspace and tape size queries, varlen planning, error strings)
with ASan and UBSan, fatal on the first report.  The ABI validation tests then
run in a child Python process that preloads the shared ASan runtime and loads
that build instead of libkda.so.  Every case in those tests fails validation
or is an empty no-op before the first HIP call, so nothing reaches a GPU.
"""
import os
import subprocess
import sys

import pytest

from hybrid_linear_attention_kda_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def sanitized_lib():
    try:
        return build.build_host_sanitized(), build.asan_runtime()
    except RuntimeError as e:  # no ROCm toolchain in this environment
        pytest.skip(str(e))


def _child_env(lib, runtime):
    env = dict(os.environ)
    pre = env.get("LD_PRELOAD", "")
    env["LD_PRELOAD"] = runtime + (":" + pre if pre else "")
    # Python itself is not instrumented: its allocations are not tracked as leaks
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0:exitcode=86"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env["KDA_LIBRARY"] = lib
    return env


def test_sanitized_build_is_instrumented(sanitized_lib):
    lib, runtime = sanitized_lib
    out = subprocess.run(["nm", "-D", lib], capture_output=True, text=True).stdout
    assert "__asan_report_load" in out and "__ubsan_handle" in out
    # and the child process really loads it
    code = "from hybrid_linear_attention_kda_amd import abi; print(abi.load()._name)"
    r = subprocess.run([sys.executable, "-c", code], env=_child_env(lib, runtime), cwd=ROOT, capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-3000:]
    assert r.stdout.strip() == lib


def test_abi_validation_under_host_sanitizers(sanitized_lib):
    lib, runtime = sanitized_lib
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi_cpu.py")],
                       env=_child_env(lib, runtime), cwd=ROOT, capture_output=True, text=True, timeout=600)
    text = r.stdout + r.stderr
    assert "AddressSanitizer" not in text and "runtime error" not in text, text[-4000:]
    assert r.returncode == 0, text[-4000:]
    assert " passed" in r.stdout
