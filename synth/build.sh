#!/bin/sh
# Builds libsynth.so (host and gfx950 device fills of the input generator) next to this script.
# Linked against PyTorch's HIP runtime, which owns the device memory and streams it fills.
set -e
here=$(cd "$(dirname "$0")" && pwd)
tlib=$(python3 -c "import importlib.util, os; print(os.path.join(os.path.dirname(importlib.util.find_spec('torch').origin), 'lib'))")
/opt/rocm/bin/hipcc --offload-arch=gfx950 -O3 -std=c++17 -fPIC -mcode-object-version=5 -ffp-contract=off \
    -Xclang -target-feature -Xclang -packed-fp32-ops \
    -c -o "$here/synth.o" "$here/synth.hip" 2>&1 | grep -v "packed-fp32-ops' is not a recognized feature" || true
test -f "$here/synth.o"
/opt/rocm/llvm/bin/clang++ -shared -o "$here/libsynth.so.tmp" "$here/synth.o" -L"$tlib" -l:libamdhip64.so \
    -Wl,-rpath,"$tlib" -Wl,--no-undefined -pthread
rm -f "$here/synth.o"
mv "$here/libsynth.so.tmp" "$here/libsynth.so"
