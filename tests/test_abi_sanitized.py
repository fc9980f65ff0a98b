"""The C-ABI layer under AddressSanitizer and UndefinedBehaviorSanitizer, on
the CPU: the host files (argument checks, the streaming driver) are rebuilt
with both sanitizers (build.build_host_sanitized), and tests/test_abi.py runs
against that library in a child process with the ASan runtime loaded first.
Any out-of-bounds access, use after free or undefined behaviour on those
paths ends the child with a sanitizer report, which fails this test."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_checks_are_clean_under_asan_and_ubsan(tmp_path):
    if os.environ.get("LD_PRELOAD"):
        pytest.skip("a preload is already set in this environment; left as it is")
    if shutil.which("g++") is None:
        pytest.skip("g++ is not available")
    asan = subprocess.run(["g++", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    if not os.path.isabs(asan) or not os.path.exists(asan):
        pytest.skip("the ASan runtime is not installed")
    sys.path.insert(0, ROOT)
    from sparse_kv_cache_gqa_amd.build import build_host_sanitized
    lib = build_host_sanitized()
    env = dict(os.environ, DA_ABI_LIB=lib, LD_PRELOAD=asan,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:exitcode=86",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1:exitcode=87")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    print(out[-4000:])
    assert "AddressSanitizer" not in out and "runtime error" not in out, "sanitizer report"
    assert r.returncode == 0, f"exit status {r.returncode}"
    assert " passed" in out
