#!/bin/bash
# Host AddressSanitizer run of the CPU test suite (no GPU needed).
#
# Builds, into a scratch directory, AddressSanitizer builds of the three host
# libraries the tests load -- the double-precision oracle (oracle/gdn_oracle.c),
# the input generator (synth/synth.c) and libgdn's host code (argument
# validation, workspace layout, planning; the device code is compiled as
# usual) -- then runs `pytest -m "not gpu"` with the sanitizer runtime
# preloaded and tests/conftest.py pointed at those builds
# (GDN_HOST_ASAN_DIR).  Any invalid host memory access aborts the run.
#
# Usage: bash tests/host_asan.sh [scratch-dir]     (from the repository root)
set -euo pipefail
ROOT=$(cd "$(dirname "$0")/.." && pwd)
OUT=${1:-/tmp/gdn_host_asan}
LLVM=/opt/rocm/lib/llvm
CLANG=$LLVM/bin/clang
RT=$(ls $LLVM/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so | head -1)
SAN="-fsanitize=address -fno-omit-frame-pointer -g -O1"
mkdir -p "$OUT"

echo "== oracle and generator (clang, host only)"
$CLANG $SAN -fPIC -shared -pthread -fno-fast-math -ffp-contract=off -o "$OUT/liboracle.so" "$ROOT/oracle/gdn_oracle.c" -lm
$CLANG $SAN -fPIC -shared -o "$OUT/libsynth.so" "$ROOT/synth/synth.c" -lm

echo "== libgdn (host code instrumented, device code as usual)"
CSRC=$ROOT/gated_delta_rule_scan_amd/csrc
HFLAGS="--offload-arch=gfx950 -O1 -g -std=c++17 -fPIC -Xclang -target-feature -Xclang -packed-fp32-ops"
HFLAGS="$HFLAGS -Xarch_host -fsanitize=address -Xarch_host -fno-omit-frame-pointer -I$ROOT/include -I$CSRC"
OBJS=""
for s in "$CSRC"/*.hip; do
  o="$OUT/$(basename "$s" .hip).o"
  /opt/rocm/bin/hipcc $HFLAGS -c "$s" -o "$o" 2>&1 | grep -v "packed-fp32" || true
  OBJS="$OBJS $o"
done
/opt/rocm/bin/hipcc --offload-arch=gfx950 -shared -fPIC -Xarch_host -fsanitize=address $OBJS -o "$OUT/libgdn.so"

echo "== pytest -m 'not gpu' under AddressSanitizer"
cd "$ROOT"
LD_PRELOAD="$RT" ASAN_OPTIONS=detect_leaks=0:alloc_dealloc_mismatch=0:abort_on_error=1 \
  GDN_HOST_ASAN_DIR="$OUT" python -m pytest tests -m "not gpu" -q -x -p no:cacheprovider
