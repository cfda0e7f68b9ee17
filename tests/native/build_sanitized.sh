#!/bin/bash
# Host AddressSanitizer + UndefinedBehaviorSanitizer builds of the library's
# argument validation (ssd_api.hip; its device code is built without them)
# and of the fp64 oracle, each linked with a driver from this folder.
# Needs the ordinary build's objects (mamba_ssd_selective_amd/_build).
# Usage: build_sanitized.sh OUTDIR   -> OUTDIR/abi_san, OUTDIR/oracle_san
set -euo pipefail
HERE="$(cd "$(dirname "$0")" && pwd)"
ROOT="$(cd "$HERE/../.." && pwd)"
OUT="$1"
OBJ="$ROOT/mamba_ssd_selective_amd/_build"
LLVM=/opt/rocm/llvm/bin
mkdir -p "$OUT"

/opt/rocm/bin/hipcc --offload-arch=gfx950 -O1 -g -std=c++17 -fPIC -Xclang -target-feature -Xclang -packed-fp32-ops -Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined -Xarch_host -fno-sanitize-recover=all -I"$ROOT/include" -c "$ROOT/mamba_ssd_selective_amd/csrc/ssd_api.hip" -o "$OUT/ssd_api_san.o" 2> "$OUT/hipcc.log" || { cat "$OUT/hipcc.log"; exit 1; }
"$LLVM/clang" -g -O1 -fsanitize=address,undefined -fno-sanitize-recover=all -I"$ROOT/include" -c "$HERE/abi_sanitize.c" -o "$OUT/abi_sanitize.o"
"$LLVM/clang++" -fsanitize=address,undefined -o "$OUT/abi_san" "$OUT/abi_sanitize.o" "$OUT/ssd_api_san.o" "$OBJ/ssd_kernels.o" "$OBJ/ssd_scan_tr.o" "$OBJ/ssd_bwd.o" "$OBJ/ssd_mixer.o" -L/opt/rocm/lib -lamdhip64 -Wl,-rpath,/opt/rocm/lib

gcc -g -O1 -fopenmp -fsanitize=address,undefined -fno-sanitize-recover=all -o "$OUT/oracle_san" "$ROOT/oracle/ssd_oracle.c" "$HERE/oracle_sanitize.c" -lm
