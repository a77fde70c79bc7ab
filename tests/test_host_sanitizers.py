"""The host-side argument checks, workspace layout and rotary table of
libblock (csrc/validate.cpp, plain C++) built with the host compiler under
AddressSanitizer and UndefinedBehaviorSanitizer and run over a table of valid,
invalid and extreme arguments (tests/host/validate_cases.cpp): every case must
give its status, and the sanitizers must report nothing (any report aborts the
run)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = [os.path.join(ROOT, "transformer_decoder_block_amd", "csrc", "validate.cpp"),
       os.path.join(ROOT, "tests", "host", "validate_cases.cpp")]


def test_validate_under_asan_ubsan(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not found")
    exe = str(tmp_path / "validate_cases")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-Wall", "-Wextra",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer", "-I", os.path.join(ROOT, "include")] + SRC + ["-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    assert "warning" not in r.stderr, r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    env.pop("LD_PRELOAD", None)
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    print(r.stdout)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "0 failed" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr
