"""Host code under AddressSanitizer + UndefinedBehaviorSanitizer (no GPU).

* ``libpfa``'s host side -- argument checks, sequence tables, the longest-first work
  schedule, workspace layouts and the plan report -- built with host-only ASan + UBSan
  (``build.py --sanitize``) and driven by ``tests/sanitize/abi_driver.cpp``: rejected
  calls of every entry point and size / plan / unit queries over 300 random tables of up
  to 128 sequences, with every host array allocated at its exact size.  That program only
  makes calls that return before anything is enqueued, so it never launches a kernel.
* The oracle (``oracle/oracle.c``) built with ASan + UBSan and driven by
  ``tests/sanitize/oracle_driver.c`` over small packed inputs of every entry point.

Any sanitizer report aborts the program, which fails the test.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
CLANG = "/opt/rocm/llvm/bin/clang++"
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1",
           "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1"}


def _run(cmd, env=None, timeout=600):
    res = subprocess.run(cmd, capture_output=True, text=True, timeout=timeout,
                         env=None if env is None else {**os.environ, **env})
    out = res.stdout + res.stderr
    print(out[-4000:])
    return res.returncode, out


@pytest.mark.skipif(not os.path.exists(CLANG), reason="ROCm clang++ not found")
def test_library_host_code_under_asan_and_ubsan(tmp_path):
    from transformer_prefill_attention_amd import build
    lib = build.build_sanitized(str(tmp_path))
    exe = str(tmp_path / "abi_driver")
    rc, out = _run([CLANG, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    "-I", os.path.join(ROOT, "include"), os.path.join(HERE, "abi_driver.cpp"),
                    "-L", str(tmp_path), "-lpfa_san", f"-Wl,-rpath,{tmp_path}", "-o", exe])
    assert rc == 0, "building the ABI driver failed"
    rc, out = _run([exe], env=SAN_ENV)
    assert rc == 0 and "abi driver: 0 failures" in out


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_oracle_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    rc, out = _run(["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    os.path.join(ROOT, "oracle", "oracle.c"), os.path.join(HERE, "oracle_driver.c"),
                    "-lm", "-lpthread", "-o", exe])
    assert rc == 0, "building the oracle driver failed"
    rc, out = _run([exe], env=SAN_ENV)
    assert rc == 0 and "oracle driver: 0 failures" in out
