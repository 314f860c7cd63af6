"""Builds libzero_shard.so (HIP for gfx950) in-tree, next to this file.

The library is linked against the HIP runtime that PyTorch ships (torch/lib),
not the system one: PyTorch owns the device memory and the streams handed to
the library, and a second HIP runtime in the same process would not see them.
"""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "csrc", "zero_shard.hip")
LIB = os.path.join(HERE, "libzero_shard.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANG = "/opt/rocm/llvm/bin/clang++"

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # Code-object v5 loads under both the system ROCm and PyTorch's bundled runtime.
    "-mcode-object-version=5",
    # The update is specified as individually rounded fp32 operations: no FMA
    # contraction, IEEE division and square root, denormals kept.
    "-ffp-contract=off",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-gpu-flush-denormals-to-zero",
    # No packed-fp32 instructions in generated code.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def torch_lib_dir() -> str:
    """Directory of PyTorch's libamdhip64.so, found without importing torch."""
    import importlib.util

    spec = importlib.util.find_spec("torch")
    if spec is None or not spec.origin:
        raise RuntimeError("PyTorch (ROCm build) is required: it supplies the HIP runtime")
    d = os.path.join(os.path.dirname(spec.origin), "lib")
    if not os.path.exists(os.path.join(d, "libamdhip64.so")):
        raise RuntimeError(f"no libamdhip64.so in {d}")
    return d


def _run(cmd) -> str:
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = ("is not a recognized feature for this target", "argument unused during compilation")
    out = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if l.strip() and not any(n in l for n in noise))
    if res.returncode != 0:
        raise RuntimeError(f"{cmd[0]} failed ({res.returncode}):\n{out}")
    return out


def build(verbose: bool = False) -> str:
    """Compile the library (always rebuilds) and return its path."""
    tlib = torch_lib_dir()
    obj = LIB + ".o"
    tmp = LIB + ".tmp"
    log = _run([HIPCC, *FLAGS, "-I", os.path.join(ROOT, "include"), "-c", "-o", obj, SRC])
    log += _run([CLANG, "-shared", "-o", tmp, obj, "-L", tlib, "-l:libamdhip64.so", f"-Wl,-rpath,{tlib}",
                 "-Wl,--no-undefined", "-lm"])
    os.remove(obj)
    if verbose and log:
        print(log)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
