"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Two programs are built for the CPU and run:
  * tests/sanitize/oracle_harness.c with oracle/attn_oracle.c (gcc): every
    oracle function on small heap arrays of exactly their stated sizes, with
    valid and rejected arguments;
  * tests/sanitize/api_harness.cpp with csrc/api.cpp (the library's host
    validation layer; clang++ from ROCm, which knows the __bf16 type of the
    shared header): every entry point with valid and rejected arguments,
    the kernel launchers replaced by stubs that check what reaches them
    (among it, the causal offset clamped to the key count).
A sanitizer report, a failed expectation or a crash fails the test.  No GPU
code is built or run.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]
CLANGXX = "/opt/rocm/llvm/bin/clang++"
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")


def _run(cmd, **kw):
    res = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert res.returncode == 0, f"{' '.join(cmd)}\n{res.stdout}\n{res.stderr}"
    return res


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_harness")
    _run(["gcc", "-std=c99", *SAN, "-Wno-unknown-pragmas",
          os.path.join(ROOT, "tests", "sanitize", "oracle_harness.c"),
          os.path.join(ROOT, "oracle", "attn_oracle.c"), "-o", exe, "-lm"])
    out = _run([exe], env=ENV)
    assert "all calls behaved" in out.stdout


@pytest.mark.skipif(not os.path.exists(CLANGXX), reason="ROCm clang++ not available")
def test_api_validation_under_sanitizers(tmp_path):
    exe = str(tmp_path / "api_harness")
    _run([CLANGXX, "-std=c++17", *SAN, "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
          "-I", os.path.join(ROOT, "include"),
          os.path.join(ROOT, "transformer_causal_self_amd", "csrc", "api.cpp"),
          os.path.join(ROOT, "tests", "sanitize", "api_harness.cpp"), "-o", exe])
    out = _run([exe], env=ENV)
    assert "all calls behaved" in out.stdout
