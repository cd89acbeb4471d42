#!/bin/bash
# The CPU test suite (-m "not gpu") with the oracle (oracle/oracle.c) and the host side of
# the C ABI library (every csrc/*.hip; device code unchanged) built under AddressSanitizer
# and UndefinedBehaviorSanitizer.  Both are built with ROCm's clang so that one sanitizer
# runtime (clang's shared libclang_rt.asan) serves the whole process; it is preloaded into
# the Python interpreter, which is not itself instrumented.  Any sanitizer report aborts
# the run (UBSan without recovery; ASan aborts on its first error).
#   usage: tests/run_sanitized.sh [output dir]   (default: a new directory under /tmp)
set -euo pipefail
ROOT=$(cd "$(dirname "$0")/.." && pwd)
OUT=${1:-$(mktemp -d /tmp/miattn_san.XXXXXX)}
mkdir -p "$OUT"
CLANG=/opt/rocm/llvm/bin/clang
RT=$("$CLANG" -print-file-name=libclang_rt.asan-x86_64.so)

"$CLANG" -O1 -g -fno-omit-frame-pointer -fsanitize=address,undefined \
    -fno-sanitize-recover=undefined -shared-libasan -fopenmp -fPIC -shared -std=c11 -Wall \
    -o "$OUT/liboracle_san.so" "$ROOT/oracle/oracle.c" -lm
python3 "$ROOT/scaled_dot_product_02_amd/build.py" --sanitize "$OUT" > /dev/null

cd "$ROOT"
# detect_leaks=0: the interpreter itself keeps allocations alive at exit
LD_PRELOAD="$RT" \
ASAN_OPTIONS=detect_leaks=0:abort_on_error=1:halt_on_error=1 \
UBSAN_OPTIONS=print_stacktrace=1:halt_on_error=1 \
ORACLE_LIB="$OUT/liboracle_san.so" MIATTN_LIB="$OUT/libmiattn_san.so" \
    python3 -m pytest tests -q -m "not gpu" -p no:cacheprovider
