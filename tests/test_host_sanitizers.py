"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Builds the oracle (gcc) and the library's host code (hipcc, sanitizers on the
host side only; the device code is compiled as usual and never runs) with
-fsanitize=address,undefined and runs a driver over every host entry point
(tests/native/).  Any invalid access, overflow or other undefined behaviour
aborts the driver.
"""
import os
import shutil
import subprocess

import pytest

from mixed_precision_adam_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
NATIVE = os.path.join(ROOT, "tests", "native")
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def _run(cmd, cwd):
    res = subprocess.run(cmd, cwd=cwd, capture_output=True, text=True, env=ENV, timeout=600)
    assert res.returncode == 0, f"{cmd[0]} failed ({res.returncode}):\n{res.stdout[-3000:]}\n{res.stderr[-3000:]}"
    return res.stdout


def test_oracle_under_sanitizers(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    exe = str(tmp_path / "oracle_checks")
    _run(["gcc", "-std=c11", "-D_DEFAULT_SOURCE", "-O1", "-g", "-ffp-contract=off", *SAN, "-o", exe,
          os.path.join(ROOT, "oracle", "oracle.c"), os.path.join(NATIVE, "oracle_checks.c"), "-lm"], tmp_path)
    assert "oracle checks ok" in _run([exe], tmp_path)


def test_library_host_code_under_sanitizers(tmp_path):
    if not os.path.exists(B.HIPCC):
        pytest.skip("hipcc not available")
    obj = str(tmp_path / "zero_shard_san.o")
    flags = [f for f in B.FLAGS if f != "-O3"] + ["-O1", "-g"]
    host_san = []
    for f in SAN:  # host side only: each sanitizer flag goes to the host compilation
        host_san += ["-Xarch_host", f]
    _run([B.HIPCC, *flags, *host_san, "-I", os.path.join(ROOT, "include"), "-c", "-o", obj, B.SRC], tmp_path)
    exe = str(tmp_path / "library_host_checks")
    tlib = B.torch_lib_dir()
    _run([B.CLANG, "-std=c++17", "-O1", "-g", *SAN, "-I", os.path.join(ROOT, "include"), "-o", exe,
          os.path.join(NATIVE, "library_host_checks.cpp"), obj, "-L", tlib, "-l:libamdhip64.so", f"-Wl,-rpath,{tlib}",
          "-lm"], tmp_path)
    assert "library host checks ok" in _run([exe], tmp_path)
