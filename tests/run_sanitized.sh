#!/bin/bash
# The CPU test suite (-m "not gpu": the oracle against its pins, the C ABI's
# argument checks, the binding's checks) with AddressSanitizer and
# UndefinedBehaviorSanitizer on the host code of the oracle and of the C ABI
# layer.  Builds liboracle_san.so and libbqmm_san.so, preloads clang's ASan
# runtime (which carries the UBSan handlers too) and runs pytest; any report
# aborts the run.  Extra arguments go to pytest.
set -euo pipefail
cd "$(dirname "$0")/.."
RT=$(/opt/rocm/llvm/bin/clang -print-file-name=libclang_rt.asan-x86_64.so)
[ -f "$RT" ] || RT=$(ls /opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so | head -1)
export BQMM_SANITIZE=1
python -c "import oracle; oracle.build(force=True)"
python -m bit_quantized_matmul_quantize_amd.build --sanitize > /dev/null
export ASAN_OPTIONS=detect_leaks=0:abort_on_error=1:halt_on_error=1
export UBSAN_OPTIONS=print_stacktrace=1:halt_on_error=1
LD_PRELOAD="$RT" python -m pytest tests -q -m "not gpu" -p no:cacheprovider "$@"
