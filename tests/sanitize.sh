#!/bin/bash
# The CPU test suite with the oracle, the input generator and the host build
# of the lane coder compiled with AddressSanitizer and UndefinedBehaviorSanitizer
# (clang; its shared runtime is preloaded into the Python process, which is not
# itself instrumented).  Runs on the CPU only; libkvc.so is not instrumented.
set -euo pipefail
cd "$(dirname "$0")/.."
RT="$(/opt/rocm/llvm/bin/clang -print-file-name=libclang_rt.asan-x86_64.so)"
export KVC_SANITIZE=1
export ASAN_OPTIONS=detect_leaks=0:abort_on_error=1:verify_asan_link_order=0
export UBSAN_OPTIONS=print_stacktrace=1:halt_on_error=1
LD_PRELOAD="$RT" python -m pytest tests -q -m "not gpu" -p no:cacheprovider "$@"
