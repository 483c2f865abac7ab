"""Host-side sanitizer builds (CPU only): the fp64 oracle and the C ABI's argument
validation, each compiled with AddressSanitizer and UndefinedBehaviorSanitizer and
driven through every index path (tests/asan/*).  An access outside a buffer or an
undefined operation aborts the driver; the drivers also check statuses, messages and
what reaches the (stubbed) launchers."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ASAN = ["-O1", "-g", "-fsanitize=address,undefined", "-fno-omit-frame-pointer", "-fno-sanitize-recover=all"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1", UBSAN_OPTIONS="halt_on_error=1",
           OMP_NUM_THREADS="3")


def _build_and_run(cmd, exe):
    res = subprocess.run(cmd, capture_output=True, text=True, cwd=ROOT)
    if res.returncode != 0 and "sanitize" in res.stderr and "unrecognized" in res.stderr:
        pytest.skip("the host compiler has no sanitizer runtime")
    assert res.returncode == 0, res.stderr
    run = subprocess.run([exe], capture_output=True, text=True, env=ENV, timeout=300)
    assert run.returncode == 0, run.stdout + run.stderr
    return run.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_oracle_under_asan(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    out = _build_and_run(["gcc", "-std=c99", "-fopenmp"] + ASAN + ["oracle/gdn_oracle.c", "tests/asan/oracle_driver.c",
                                                                   "-lm", "-o", exe], exe)
    assert "all checks passed" in out


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not found")
def test_abi_validation_under_asan(tmp_path):
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    if not os.path.exists(os.path.join(rocm, "include", "hip", "hip_runtime_api.h")):
        pytest.skip("HIP headers not found")
    exe = str(tmp_path / "validation_driver")
    out = _build_and_run(["g++", "-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(rocm, "include"),
                          "-I", "include", "-I", "gated_deltanet_rule_amd/csrc"] + ASAN +
                         ["gated_deltanet_rule_amd/csrc/gdn_api.cpp", "tests/asan/validation_driver.cpp", "-o", exe],
                         exe)
    assert "all checks passed" in out
