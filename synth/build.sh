#!/bin/sh
# Builds libsynth.so (host and gfx950 device fills of the input generator) next to this script.
set -e
here=$(cd "$(dirname "$0")" && pwd)
/opt/rocm/bin/hipcc --offload-arch=gfx950 -O3 -std=c++17 -fPIC -shared -ffp-contract=off \
    -Xclang -target-feature -Xclang -packed-fp32-ops -pthread \
    -o "$here/libsynth.so.tmp" "$here/synth.hip" 2>&1 | grep -v "packed-fp32-ops' is not a recognized feature" || true
test -f "$here/libsynth.so.tmp"
mv "$here/libsynth.so.tmp" "$here/libsynth.so"
