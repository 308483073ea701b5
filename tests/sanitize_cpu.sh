#!/bin/bash
# AddressSanitizer + UndefinedBehaviorSanitizer runs of the CPU-side code, in a
# machine without a GPU:
#   1. the C oracle (oracle/gdn_oracle.c) built with gcc's sanitizers, under
#      tests/test_oracle_pins.py;
#   2. the host code of libgdn.so (argument checks, workspace layout, launch
#      set-up in every .hip file) built with clang's sanitizers on the host
#      side only, under tests/test_abi_host.py.
# Usage: bash tests/sanitize_cpu.sh [build dir]   (default _build/sanitize)
set -euo pipefail
ROOT=$(cd "$(dirname "$0")/.." && pwd)
OUT=${1:-$ROOT/_build/sanitize}
mkdir -p "$OUT"
cd "$ROOT"
export ASAN_OPTIONS=detect_leaks=0:abort_on_error=1:halt_on_error=1
export UBSAN_OPTIONS=print_stacktrace=1:halt_on_error=1

echo "== oracle with gcc -fsanitize=address,undefined"
gcc -O1 -g -fno-omit-frame-pointer -fsanitize=address,undefined -fno-sanitize-recover=undefined \
    -fopenmp -fPIC -shared -std=c99 -o "$OUT/liboracle_san.so" oracle/gdn_oracle.c
LD_PRELOAD="$(gcc -print-file-name=libasan.so)" GDN_ORACLE_LIB="$OUT/liboracle_san.so" \
    python -m pytest -q -m "not gpu" -p no:cacheprovider tests/test_oracle_pins.py

echo "== libgdn.so host code with clang -fsanitize=address,undefined (host side only)"
HIPCC=${HIPCC:-/opt/rocm/bin/hipcc}
FLAGS=(--offload-arch=gfx950 -O1 -g -std=c++17 -fPIC -fno-omit-frame-pointer
       -Xclang -target-feature -Xclang -packed-fp32-ops
       -Iinclude -Ihybrid_linear_attention_amd/csrc)
OBJS=()
for src in gdn_api gdn_attention gdn_backward gdn_decode gdn_prefill; do
  $HIPCC "${FLAGS[@]}" -Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined \
      -Xarch_host -fno-sanitize-recover=undefined \
      -c "hybrid_linear_attention_amd/csrc/$src.hip" -o "$OUT/$src.o" 2>&1 | grep -v packed-fp32 || true
  OBJS+=("$OUT/$src.o")
done
$HIPCC --offload-arch=gfx950 -shared -fPIC -shared-libsan -Xarch_host -fsanitize=address \
    -Xarch_host -fsanitize=undefined -o "$OUT/libgdn_san.so" "${OBJS[@]}"
RT=$($HIPCC -print-file-name=libclang_rt.asan-x86_64.so)
LD_PRELOAD="$RT" GDN_LIB_PATH="$OUT/libgdn_san.so" \
    python -m pytest -q -m "not gpu" -p no:cacheprovider tests/test_abi_host.py
echo "== sanitizer runs clean"
