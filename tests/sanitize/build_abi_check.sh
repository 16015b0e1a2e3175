#!/bin/bash
# Host-sanitized build of the library (device code as usual: every sanitizer
# flag goes to the host pass only) and of the ABI driver that calls it.
# Usage: build_abi_check.sh OUT_DIR
set -e
OUT=$1
ROOT=$(cd "$(dirname "$0")/../.." && pwd)
CS=$ROOT/non_prefix_kv_token_amd/csrc
mkdir -p "$OUT"
HF="-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined -Xarch_host -fno-sanitize-recover=all -Xarch_host -fno-omit-frame-pointer"
F="--offload-arch=gfx950 -O1 -g -fPIC -std=c++17 -Xclang -target-feature -Xclang -packed-fp32-ops -I$ROOT/include -I$CS"
OBJS=""
for f in abi score topr assemble attn attn_f32 timing hosttier layer; do
  /opt/rocm/bin/hipcc $F $HF -c $CS/$f.hip -o "$OUT/$f.o" &
  OBJS="$OBJS $OUT/$f.o"
done
/opt/rocm/bin/hipcc $F $HF -c $CS/calibrate.cpp -o "$OUT/calibrate.o" &
wait
/opt/rocm/bin/hipcc --offload-arch=gfx950 -shared -fPIC $HF $OBJS "$OUT/calibrate.o" -o "$OUT/libcachetune_asan.so"
/opt/rocm/llvm/bin/clang -O1 -g -fsanitize=address,undefined -fno-sanitize-recover=all -fno-omit-frame-pointer -D__HIP_PLATFORM_AMD__ \
  -I$ROOT/include -I/opt/rocm/include "$ROOT/tests/sanitize/abi_check.c" "$OUT/libcachetune_asan.so" \
  -Wl,-rpath,"$OUT" -L/opt/rocm/lib -lamdhip64 -lm -o "$OUT/abi_check"
