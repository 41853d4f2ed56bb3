"""The host-side code -- the C ABI's validation and planning, the hybrid step's
CPU attention, and the oracle -- under AddressSanitizer and
UndefinedBehaviorSanitizer: the CPU test suites run again in a child process
against clang-built, host-instrumented copies of both libraries, with the
sanitizer runtime preloaded.  Device code is not instrumented (CPU only)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLANG = "/opt/rocm/llvm/bin/clang"


def test_cpu_suites_clean_under_asan_and_ubsan():
    if not os.path.exists(CLANG):
        pytest.skip("clang of the ROCm toolchain not found")
    rt = subprocess.check_output([CLANG, "-print-file-name=libclang_rt.asan-x86_64.so"], text=True).strip()
    if not os.path.isabs(rt) or not os.path.exists(rt):
        pytest.skip("clang's AddressSanitizer runtime not found")
    sys.path.insert(0, ROOT)
    from oracle import oracle
    from sparse_kv_cache_block_amd import build
    skv_lib = build.build(sanitize=True)
    orc_lib = oracle.build_sanitized()
    env = dict(os.environ, LD_PRELOAD=rt, SKV_LIB=skv_lib, SKV_ORACLE_LIB=orc_lib,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    suites = ["tests/test_abi_cpu.py", "tests/test_host_attention.py", "tests/test_oracle_pins.py",
              "tests/test_inputs.py"]
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-m", "not gpu", "-p", "no:cacheprovider", *suites],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=1200)
    report = r.stdout[-4000:] + r.stderr[-4000:]
    assert r.returncode == 0, report
    assert "AddressSanitizer" not in report and "runtime error" not in report, report
