"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

The argument checks, plans, workspace sizing, metadata checkers, block manager
and scheduler (pa_host.cpp, pa_api.cpp, pa_runtime.cpp) are built with g++ and
-fsanitize=address,undefined as a host-only library of the same ABI (kernel
launches replaced by a "no device" error), and the ABI and runtime test files
run against it in a child process with the ASan runtime preloaded.  Any
sanitizer report fails the test.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _runtime(name):
    r = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True)
    path = r.stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


@pytest.mark.skipif(_runtime("libasan.so") is None, reason="gcc's ASan runtime is not installed")
def test_abi_and_runtime_tests_pass_under_asan_and_ubsan():
    from paged_kv_attention_13_amd import build
    lib = build.build_host_only(sanitize=True)
    env = dict(os.environ)
    pre = env.get("LD_PRELOAD", "")
    env["LD_PRELOAD"] = _runtime("libasan.so") + (":" + pre if pre else "")
    # the interpreter and torch are not instrumented: leak checking and the allocator
    # pairing check would report their memory, not the library's
    env["ASAN_OPTIONS"] = "detect_leaks=0:alloc_dealloc_mismatch=0:halt_on_error=1:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env["PA_LIB_PATH"] = lib
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
           os.path.join(ROOT, "tests", "test_abi.py"), os.path.join(ROOT, "tests", "test_runtime.py")]
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    log = r.stdout[-4000:] + r.stderr[-4000:]
    assert r.returncode == 0, log
    assert "AddressSanitizer" not in r.stderr and "runtime error:" not in r.stderr, log
    assert " passed" in r.stdout, log
    # the child really ran against the sanitizer build
    assert "libpa_host_san.so" in lib
