#!/bin/sh
# Builds the CPU oracle (test infrastructure) as a shared library next to this script.
# Plain single-threaded C: no contraction of a*b+c, no fast-math, SSE2 floating point.
# Optional arguments: source file and output library (defaults: oracle.c and liboracle.so here); the test
# that plants mistakes in a copy of the oracle builds the copy with the same flags this way.
set -e
here=$(cd "$(dirname "$0")" && pwd)
src=${1:-$here/oracle.c}
out=${2:-$here/liboracle.so}
gcc -std=c11 -D_DEFAULT_SOURCE -O2 -ffp-contract=off -fno-fast-math -fno-tree-vectorize -fPIC -shared \
    -Wall -Wextra -I "$here" -o "$out.tmp" "$src" -lm
mv "$out.tmp" "$out"
