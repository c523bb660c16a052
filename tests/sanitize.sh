#!/bin/bash
# CPU sanitizer run: the fp64 oracle (gcc, AddressSanitizer + UndefinedBehaviorSanitizer) under its pin
# tests, and the host side of libpathattn (clang, the same sanitizers on host code only; device code is
# built as usual) under the host-side ABI tests.  Two processes, one sanitizer runtime each.  No GPU is
# used: every ABI test fails validation (or is a pure host query) before anything is enqueued.
# Usage: tests/sanitize.sh   (from the repository root; builds into _build/sanitize)
set -euo pipefail
ROOT=$(cd "$(dirname "$0")/.." && pwd)
OUT=$ROOT/_build/sanitize
mkdir -p "$OUT"
export ASAN_OPTIONS=detect_leaks=0:abort_on_error=1
export UBSAN_OPTIONS=halt_on_error=1:print_stacktrace=1

echo "[sanitize] oracle: gcc -fsanitize=address,undefined"
gcc -O1 -g -fno-omit-frame-pointer -fsanitize=address,undefined -fno-sanitize-recover=undefined -std=c11 -fPIC \
  -shared -pthread -Wall -Wextra -fno-fast-math -o "$OUT/libpathoracle_san.so" "$ROOT/oracle/path_oracle.c" -lm
( cd "$ROOT" && PATHORACLE_LIB="$OUT/libpathoracle_san.so" \
  LD_PRELOAD="$(gcc -print-file-name=libasan.so):$(gcc -print-file-name=libubsan.so)" \
  python -m pytest -x -q -m "not gpu" -p no:cacheprovider tests/test_oracle_pins.py )

echo "[sanitize] libpathattn host code: hipcc -Xarch_host -fsanitize=address,undefined"
HIPCC=/opt/rocm/bin/hipcc
objs=()
for f in "$ROOT"/dependent_positional_attention_amd/csrc/*.hip; do
  o="$OUT/$(basename "$f").o"
  $HIPCC --offload-arch=gfx950 -O1 -g -std=c++17 -fPIC -I "$ROOT/include" \
    -I "$ROOT/dependent_positional_attention_amd/csrc" -Xclang -target-feature -Xclang -packed-fp32-ops \
    -mllvm --disable-promote-alloca-to-lds -Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined \
    -Xarch_host -fno-omit-frame-pointer -c "$f" -o "$o" 2>&1 | grep -v "packed-fp32" || true
  objs+=("$o")
done
$HIPCC --offload-arch=gfx950 -shared -fPIC -Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined \
  -o "$OUT/libpathattn_san.so" "${objs[@]}"
CLANG_RT=$(ls /opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so | head -1)
( cd "$ROOT" && PATHATTN_LIB="$OUT/libpathattn_san.so" LD_PRELOAD="$CLANG_RT" \
  python -m pytest -x -q -m "not gpu" -p no:cacheprovider tests/test_abi.py tests/test_zz_no_alloc.py )
echo "[sanitize] clean"
