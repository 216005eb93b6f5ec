#!/bin/bash
# Builds the host side of libspecattn with AddressSanitizer and
# UndefinedBehaviorSanitizer (device code unchanged; -Xarch_host keeps the
# sanitizers on the host pass) plus the debug plan checker, links the
# abi_driver against it, and runs the driver on the CPU.  Needs the regular
# build's objects in _build/ (python -m sparse_kv_attention_sink_amd.build).
set -euo pipefail
R="$(cd "$(dirname "$0")/../.." && pwd)"
O="$R/_build/sanitize"
C="$R/sparse_kv_attention_sink_amd/csrc"
mkdir -p "$O"
HIPCC="${HIPCC:-/opt/rocm/bin/hipcc}"
CLANG="${CLANG:-/opt/rocm/llvm/bin/clang}"
"$HIPCC" --offload-arch=gfx950 -O1 -g -std=c++17 -fPIC -DSPEC_DEBUG_PLAN \
  -Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined \
  -Xarch_host -fno-sanitize-recover=undefined -Xarch_host -fno-omit-frame-pointer \
  -Xclang -target-feature -Xclang -packed-fp32-ops \
  -I "$R/include" -I "$C" -c "$C/api.hip" -o "$O/api_asan.o" 2> "$O/api.log"
"$CLANG" -O1 -g -fsanitize=address,undefined -fno-sanitize-recover=undefined -fno-omit-frame-pointer \
  -Wall -Werror -I "$R/include" -I "$R/tests/sanitize" -c "$R/tests/sanitize/abi_driver.c" -o "$O/driver.o"
"$HIPCC" --offload-arch=gfx950 -Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined \
  "$O/driver.o" "$O/api_asan.o" "$R/_build/attn.o" "$R/_build/generic.o" "$R/_build/accept.o" \
  "$R/_build/commit.o" "$R/_build/select.o" "$R/_build/gather.o" -o "$O/abi_driver" 2> "$O/link.log"
ASAN_OPTIONS=detect_leaks=0:abort_on_error=0:halt_on_error=1 UBSAN_OPTIONS=print_stacktrace=1 "$O/abi_driver"
