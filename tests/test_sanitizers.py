"""CPU-only: the oracle (oracle/oracle.c) and the C ABI's host-side argument
checks (csrc/validate.cpp) built with AddressSanitizer and
UndefinedBehaviorSanitizer (gcc, runtime linked statically, every finding
fatal), each driven over valid, invalid and extreme arguments by a small
program under tests/sanitize/.  A finding aborts the program and fails the
test with the sanitizer's report."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
SAN = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
       "-fno-sanitize-recover=all", "-static-libasan", "-static-libubsan"]

BUILDS = {
    "oracle": ["gcc", "-std=c11", "-ffp-contract=off", *SAN, "-I", os.path.join(ROOT, "oracle"),
               os.path.join(HERE, "oracle_driver.c"), os.path.join(ROOT, "oracle", "oracle.c"),
               "-lm"],
    "validate": ["g++", "-std=c++17", *SAN, "-I", os.path.join(ROOT, "include"),
                 "-I", os.path.join(ROOT, "bit_quantized_decode_amd", "csrc"),
                 os.path.join(HERE, "validate_driver.cpp"),
                 os.path.join(ROOT, "bit_quantized_decode_amd", "csrc", "validate.cpp")],
}


@pytest.mark.parametrize("name", sorted(BUILDS))
def test_clean_under_asan_and_ubsan(tmp_path, name):
    exe = str(tmp_path / f"{name}_driver")
    subprocess.run(BUILDS[name] + ["-o", exe], check=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0 and "done" in r.stdout, r.stdout + r.stderr
