"""CPU runs under AddressSanitizer and UndefinedBehaviorSanitizer.

  * the fp64 oracle (oracle/*.c), every entry on small inputs, built with gcc;
  * the host code of the HIP library (argument validation, the tile table,
    workspace sizes, status text), built with hipcc with the sanitizers on the
    host pass only; every call is rejected before any HIP call, so no GPU is
    needed.

A sanitizer report, a leak in the oracle run, or a failed check is a failure.
"""
from __future__ import annotations

import os
import shutil
import subprocess
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parent.parent
SAN = ROOT / "tests" / "sanitize"
CSRC = ROOT / "attention_flashattention_fwd_amd" / "csrc"
ENV = {**os.environ,
       "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
       "OMP_NUM_THREADS": "2"}


def run(exe: Path, leaks: bool):
    env = {**ENV, "ASAN_OPTIONS": f"halt_on_error=1:detect_leaks={int(leaks)}"}
    res = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300, env=env)
    report = res.stdout + res.stderr
    assert res.returncode == 0, report
    assert "runtime error" not in report and "AddressSanitizer" not in report, report
    return report


def test_oracle_under_sanitizers(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not found")
    exe = tmp_path / "oracle_checks"
    cmd = ["gcc", "-O1", "-g", "-fsanitize=address,undefined", "-fno-omit-frame-pointer",
           "-fopenmp", "-std=c99", str(SAN / "oracle_checks.c"),
           *sorted(str(p) for p in (ROOT / "oracle").glob("*.c")), "-o", str(exe), "-lm"]
    subprocess.run(cmd, check=True, capture_output=True, timeout=300)
    assert "oracle checks: ok" in run(exe, leaks=True)


def test_library_host_code_under_sanitizers(tmp_path):
    from attention_flashattention_fwd_amd import build

    exe = tmp_path / "abi_checks"
    # the sanitizers go to the host pass only (the GPU code is never run here)
    cmd = [build.hipcc(), "--offload-arch=gfx950", "-O1", "-g", "-std=c++20", "-fno-honor-nans",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-omit-frame-pointer",
           f"-I{ROOT / 'include'}", f"-I{CSRC}",
           *(str(p) for p in build.SOURCES), str(SAN / "abi_checks.cpp"), "-o", str(exe)]
    res = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert res.returncode == 0, res.stderr[-3000:]
    # leak checking is off here: the HIP runtime keeps allocations until exit
    assert "abi checks: ok" in run(exe, leaks=False)
