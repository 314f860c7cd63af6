"""The C ABI from plain C on the GPU: tests/c_abi/rank_step.c, compiled with gcc against include/zero_shard.h
and the HIP runtime's C API (no PyTorch in that process), runs one rank's step twice (host decision, then
device decision) and compares every result with the oracle; it exits 0 only if all agree."""
import os
import shutil
import subprocess

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_rank_step_from_plain_c(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    exe = str(tmp_path / "rank_step")
    libdirs = [os.path.join(ROOT, d) for d in ("mixed_precision_adam_amd", "oracle", "synth")] + ["/opt/rocm/lib"]
    cmd = ["gcc", "-std=c11", "-O1", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "oracle"), "-I", os.path.join(ROOT, "synth"),
           os.path.join(ROOT, "tests", "c_abi", "rank_step.c"), "-o", exe]
    for d in libdirs:
        cmd += ["-L", d, f"-Wl,-rpath,{d}"]
    cmd += ["-l:libzero_shard.so", "-l:liboracle.so", "-l:libsynth.so", "-lamdhip64", "-lm"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    print("[c-abi] built, running", flush=True)
    res = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "all equal to the oracle" in res.stdout
