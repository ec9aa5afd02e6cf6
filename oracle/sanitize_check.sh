#!/bin/bash
# Runs the oracle's pin suite (tests/test_oracle_pins.py) against a build of
# ksa_oracle.c with AddressSanitizer and UndefinedBehaviorSanitizer (gcc, host
# code only; the runtimes are preloaded into the Python process that loads
# the oracle through ctypes).  Any sanitizer report fails the run.
set -euo pipefail
cd "$(dirname "$0")/.."
dir=$(mktemp -d)
trap 'rm -rf "$dir"' EXIT
lib="$dir/libksa_oracle_san.so"
gcc -O1 -g -std=c11 -fPIC -shared -fopenmp -fno-fast-math -ffp-contract=off -Wall -Wextra \
    -fsanitize=address,undefined -fno-sanitize-recover=all -fno-omit-frame-pointer \
    -o "$lib" oracle/ksa_oracle.c -lm
export LD_PRELOAD="$(gcc -print-file-name=libasan.so) $(gcc -print-file-name=libubsan.so)"
export ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1"
export UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1"
export KSA_ORACLE_LIB="$lib"
python -m pytest tests/test_oracle_pins.py -q -p no:cacheprovider "$@"
