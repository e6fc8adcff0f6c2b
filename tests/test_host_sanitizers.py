"""The host side of liblra (argument validation, workspace layouts, launch set-up) under
AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

The library is rebuilt with its host code instrumented (``build.py --sanitize``: every
``-fsanitize=`` is given to the host compilation only, the gfx950 code is built as usual) and
``tests/test_abi.py`` runs against it in a child process with the ASan runtime preloaded. Every call
in that file fails validation before anything is enqueued, so no GPU is needed; any invalid memory
access or undefined behaviour in the host code aborts the child and fails this test.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, os.path.join(ROOT, "rank_kv_cache_amd"))
import build as lra_build  # noqa: E402  (the package's build script, imported without loading liblra)


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="hipcc is required to build the sanitized library")
def test_abi_suite_clean_under_asan_and_ubsan():
    lib = lra_build.build_sanitized(verbose=False)
    undefined = subprocess.run(["nm", "-D", "--undefined-only", lib], capture_output=True, text=True).stdout
    assert "__asan_" in undefined and "__ubsan_" in undefined, "the host code is not instrumented"
    env = dict(os.environ)
    env.update({
        "LD_PRELOAD": lra_build.sanitizer_runtime(),
        "LRA_LIB_PATH": lib,
        # the interpreter and torch are not instrumented: no leak report at exit, and no allocator
        # mismatch or ODR checks across their libraries
        "ASAN_OPTIONS": "detect_leaks=0:alloc_dealloc_mismatch=0:detect_odr_violation=0:abort_on_error=1",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
    })
    check = "import rank_kv_cache_amd as l; assert l.LIB_PATH == %r, l.LIB_PATH" % lib
    r = subprocess.run([sys.executable, "-c", check], cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "tests/test_abi.py"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert " passed" in out
