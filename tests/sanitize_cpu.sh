#!/bin/bash
# CPU-only sanitizer run: builds the oracle (clang, -fsanitize=address,undefined)
# and the host side of libprox (hipcc, -Xarch_host -fsanitize=address and
# undefined; device code is built as usual) in a scratch copy of the repository,
# then runs the CPU test suite (-m "not gpu") there with the ASan runtime
# preloaded.  Usage: bash tests/sanitize_cpu.sh [extra pytest args]
set -euo pipefail
REPO=$(cd "$(dirname "$0")/.." && pwd)
WORK=$(mktemp -d /tmp/prox_san.XXXXXX)
trap 'rm -rf "$WORK"' EXIT
LLVM=/opt/rocm/llvm
ASAN_RT=$(ls "$LLVM"/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so | head -n 1)
mkdir -p "$WORK/free_sparse_swiglu_amd"
cp -r "$REPO/oracle" "$REPO/tests" "$REPO/include" "$WORK/"
cp -r "$REPO/free_sparse_swiglu_amd/csrc" "$WORK/free_sparse_swiglu_amd/"
cp "$REPO"/free_sparse_swiglu_amd/*.py "$WORK/free_sparse_swiglu_amd/"
rm -f "$WORK"/oracle/*.so
cd "$WORK"
SAN="-fsanitize=address,undefined -fno-sanitize-recover=undefined -fno-omit-frame-pointer"
python -c "import sys; sys.path.insert(0, '.'); from oracle import prox_oracle as o; \
o.build(force=True, cc='$LLVM/bin/clang', extra_flags='$SAN'.split())"
python free_sparse_swiglu_amd/build.py --sanitize > build.log 2>&1
nm -D oracle/libprox_oracle.so | grep -q __asan_
nm -D free_sparse_swiglu_amd/libprox.so | grep -q __ubsan_
export ASAN_OPTIONS=detect_leaks=0:abort_on_error=1:halt_on_error=1
export UBSAN_OPTIONS=print_stacktrace=1:halt_on_error=1
LD_PRELOAD="$ASAN_RT" python -m pytest tests -q -m "not gpu" -p no:cacheprovider "$@"
