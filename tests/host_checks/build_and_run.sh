#!/bin/bash
# Build the library's sources (device code as usual, host code with
# AddressSanitizer and UndefinedBehaviorSanitizer) with the host-check driver
# and run it.  usage: build_and_run.sh OUTDIR
set -euo pipefail
here=$(cd "$(dirname "$0")" && pwd)
root=$(cd "$here/../.." && pwd)
out=${1:-$root/_build/host_checks}
mkdir -p "$out"
csrc=$root/mixture_experts_layer_mk_amd/csrc
hipcc=${HIPCC:-/opt/rocm/bin/hipcc}
common=(-O1 -g -std=c++17 -I"$root/include" -I"$csrc")
objs=()
pids=()
for f in "$csrc"/*.hip; do
  o="$out/$(basename "$f" .hip).o"
  objs+=("$o")
  "$hipcc" --offload-arch=gfx950 "${common[@]}" -Xclang -target-feature -Xclang -packed-fp32-ops \
    -Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined \
    -Xarch_host -fno-omit-frame-pointer -Xarch_host -fno-sanitize-recover=all \
    -c "$f" -o "$o" 2> "$o.log" &
  pids+=($!)
done
for p in "${pids[@]}"; do wait "$p"; done
"$hipcc" -x c++ "${common[@]}" -Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined \
  -Xarch_host -fno-sanitize-recover=all -fno-omit-frame-pointer \
  -c "$here/host_checks.cpp" -o "$out/host_checks.o"
"$hipcc" --offload-arch=gfx950 -Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined \
  "$out/host_checks.o" "${objs[@]}" -o "$out/host_checks"
ASAN_OPTIONS=detect_leaks=0:abort_on_error=0 UBSAN_OPTIONS=print_stacktrace=1:halt_on_error=1 \
  "$out/host_checks"
