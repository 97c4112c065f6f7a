#!/bin/bash
# The CPU test suite (-m "not gpu") under AddressSanitizer and
# UndefinedBehaviorSanitizer: the oracle (oracle/tvref.c) and the host side of
# libtv.so (include/tree_verify.h's C ABI in tv_api.cpp: argument checks,
# planner, workspace sizes; launches stubbed by host_stubs.cpp) are built
# with gcc / g++ and both sanitizers, and the tests load them through
# TVREF_LIB and TV_LIB. Host compilers only: no GPU code is built or run.
# Extra arguments go to pytest.
set -euo pipefail
ROOT=$(cd "$(dirname "$0")/../.." && pwd)
OUT=$ROOT/_build/sanitize
mkdir -p "$OUT"
SAN="-fsanitize=address,undefined -fno-sanitize-recover=undefined -fno-omit-frame-pointer -g -O1"
gcc -std=c11 -ffp-contract=off -fopenmp -shared -fPIC $SAN "$ROOT/oracle/tvref.c" -o "$OUT/libtvref.so" -lm
g++ -std=c++17 -shared -fPIC $SAN -D__HIP_PLATFORM_AMD__ -I/opt/rocm/include -I"$ROOT/include" \
    -I"$ROOT/tree_verify_attention_ddtree_amd/csrc" "$ROOT/tree_verify_attention_ddtree_amd/csrc/tv_api.cpp" \
    "$ROOT/tests/sanitize/host_stubs.cpp" -L/opt/rocm/lib -lamdhip64 -Wl,-rpath,/opt/rocm/lib -o "$OUT/libtv_host.so"
PRE="$(gcc -print-file-name=libasan.so):$(gcc -print-file-name=libubsan.so)"
cd "$ROOT"
LD_PRELOAD="$PRE" ASAN_OPTIONS=detect_leaks=0:abort_on_error=1 UBSAN_OPTIONS=print_stacktrace=1:halt_on_error=1 \
    TV_LIB="$OUT/libtv_host.so" TVREF_LIB="$OUT/libtvref.so" \
    python -m pytest tests -q -m "not gpu" -p no:cacheprovider "$@"
