"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Two programs are built with gcc / g++ and `-fsanitize=address,undefined
-fno-sanitize-recover=all`, so that any out-of-bounds access, leak or
undefined operation fails the run:
  * tests/sanitize/oracle_driver.c with oracle/dsa_oracle.c: every oracle
    function on small inputs and edge cases (empty rows, k above n_valid,
    masked, out-of-range and duplicate entries, zero and huge FP8 blocks);
  * tests/sanitize/api_driver.cpp with sparse_attention_amd/csrc/dsa_api.cpp
    and the real launch planning (launch_plan.h), the kernel launchers
    replaced by host stand-ins (tests/sanitize/api_stubs.cpp): validation,
    workspace sizing and layout of every C entry point, including size
    queries with extreme arguments and decode-step structs allocated with
    only the fields their struct_size declares.
Only host code is built; no GPU code is compiled with a sanitizer.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1",
           OMP_NUM_THREADS="2")


def _build(tmp_path, compiler, out, sources, extra=()):
    if shutil.which(compiler) is None:
        pytest.skip("%s not available" % compiler)
    exe = str(tmp_path / out)
    cmd = [compiler, *SAN, *extra, "-o", exe, *sources]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, "build failed: %s\n%s" % (" ".join(cmd), r.stderr)
    return exe


def _run(exe):
    r = subprocess.run([exe], capture_output=True, text=True, env=ENV, timeout=300)
    assert r.returncode == 0 and "runtime error" not in r.stderr and "Sanitizer" not in r.stderr, \
        "sanitizer run failed (%d):\n%s\n%s" % (r.returncode, r.stdout, r.stderr[-4000:])
    return r.stdout


def test_oracle_under_sanitizers(tmp_path):
    exe = _build(tmp_path, "gcc", "oracle_driver",
                 [os.path.join(ROOT, "tests", "sanitize", "oracle_driver.c"), os.path.join(ROOT, "oracle", "dsa_oracle.c")],
                 ["-std=c99", "-fopenmp", "-lm"])
    assert "oracle driver: ok" in _run(exe)


def test_c_abi_host_code_under_sanitizers(tmp_path):
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    exe = _build(tmp_path, "g++", "api_driver",
                 [os.path.join(ROOT, "tests", "sanitize", "api_driver.cpp"),
                  os.path.join(ROOT, "tests", "sanitize", "api_stubs.cpp"),
                  os.path.join(ROOT, "sparse_attention_amd", "csrc", "dsa_api.cpp")],
                 ["-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(rocm, "include"),
                  "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "sparse_attention_amd", "csrc")])
    out = _run(exe)
    assert "api driver:" in out and out.strip().endswith("ok")
