"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Two host-only executables are built with gcc/g++ (no GPU code in either):
  * the CPU oracle (oracle/lq_oracle.c) with a driver that calls every entry
    point on small inputs and the degenerate cases;
  * the library's C ABI layer (csrc/lq_api.hip, compiled as plain C++) with
    the kernel launchers stubbed, so that every entry point's argument checks
    and the blob layout run.
Any sanitizer report aborts the run (-fno-sanitize-recover=all).
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1",
           OMP_NUM_THREADS="2")


def _run(cmd, cwd):
    r = subprocess.run(cmd, cwd=cwd, capture_output=True, text=True, timeout=300, env=ENV)
    assert r.returncode == 0, (cmd, r.stdout[-3000:], r.stderr[-3000:])
    return r.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = tmp_path / "oracle_driver"
    _run(["gcc", "-std=c11", *SAN, "-fopenmp", os.path.join(ROOT, "tests", "sanitize", "oracle_driver.c"),
          os.path.join(ROOT, "oracle", "lq_oracle.c"), "-o", str(exe), "-lm"], ROOT)
    out = _run([str(exe)], ROOT)
    assert "all calls returned 0" in out


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"),
                    reason="needs g++ and the HIP headers")
def test_abi_validation_under_asan_ubsan(tmp_path):
    exe = tmp_path / "abi_validation"
    csrc = os.path.join(ROOT, "linear_attention_recurrent_gdn_amd", "csrc")
    _run(["g++", "-std=c++17", *SAN, "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
          f"-I{os.path.join(ROOT, 'include')}", f"-I{csrc}",
          "-x", "c++", os.path.join(csrc, "lq_api.hip"),
          "-x", "c++", os.path.join(ROOT, "tests", "sanitize", "abi_validation.cpp"), "-o", str(exe)], ROOT)
    out = _run([str(exe)], ROOT)
    assert "all checks passed" in out
