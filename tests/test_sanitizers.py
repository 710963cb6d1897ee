"""CPU builds of the host code under AddressSanitizer and
UndefinedBehaviorSanitizer (the GPU kernels are not part of them):

* the fp64 oracle (oracle/rehyat_oracle.c) over tiny geometries of every
  feature map and both partitions, with row subsets, partials, invalid
  arguments and the non-finite report (tests/native/oracle_sanitize_check.c);
* the library's host side (csrc/api.cpp: validation, geometry, workspace
  sizing, step-state header, error strings, fault injection) driven through
  every entry point with the kernel launchers stubbed out
  (tests/native/host_sanitize_check.cpp).  Every call there either fails
  validation or stops at its first HIP step (fault-injection hook), so no GPU
  is touched."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
NATIVE = os.path.join(ROOT, "tests", "native")
CSRC = os.path.join(ROOT, "linear_attention_video_rehyat_amd", "csrc")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-g", "-O1"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")


def _run(cmd, **kw):
    res = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert res.returncode == 0, (" ".join(cmd) + "\n" + res.stdout[-3000:] + res.stderr[-3000:])
    return res


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_sanitize_check")
    _run(["gcc", "-std=c11", "-fopenmp", *SAN, os.path.join(NATIVE, "oracle_sanitize_check.c"),
          os.path.join(ROOT, "oracle", "rehyat_oracle.c"), "-lm", "-o", exe])
    res = _run([exe], env=dict(ENV, OMP_NUM_THREADS="2"), timeout=300)
    assert " 0 failures" in res.stdout and "runtime error" not in res.stderr


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.exists("/opt/rocm/lib/libamdhip64.so"),
                    reason="g++ or the HIP runtime library not available")
def test_host_validation_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "host_sanitize_check")
    _run(["g++", "-std=c++17", *SAN, "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", f"-I{CSRC}",
          os.path.join(NATIVE, "host_sanitize_check.cpp"), os.path.join(CSRC, "api.cpp"),
          "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", exe])
    res = _run([exe], env=ENV, timeout=300)
    assert " 0 failures" in res.stdout and "runtime error" not in res.stderr
