#!/bin/sh
# Builds the CPU oracle (test infrastructure) as a shared library next to this script.
# Plain single-threaded C: no contraction of a*b+c, no fast-math, SSE2 floating point.
set -e
here=$(cd "$(dirname "$0")" && pwd)
gcc -std=c11 -D_DEFAULT_SOURCE -O2 -ffp-contract=off -fno-fast-math -fno-tree-vectorize -fPIC -shared \
    -Wall -Wextra -o "$here/liboracle.so.tmp" "$here/oracle.c" -lm
mv "$here/liboracle.so.tmp" "$here/liboracle.so"
