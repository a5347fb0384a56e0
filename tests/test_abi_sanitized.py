"""The host side of the C ABI (argument validation, planning, workspace
sizing) under AddressSanitizer and UndefinedBehaviorSanitizer: the library
is rebuilt with both on its host code and tests/test_abi.py runs against it
in a child Python with the ASan runtime preloaded.  Any sanitizer report
fails the child (undefined behaviour aborts; ASan aborts by default)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, os.path.join(ROOT, "tests", "sanitize"))

import build_sanitized  # noqa: E402


def test_abi_checks_under_sanitizers():
    lib = build_sanitized.build()
    env = dict(os.environ)
    env["LD_PRELOAD"] = build_sanitized.runtime()
    env["DDT_ABI_TEST_LIB"] = lib
    # leak checking would report the interpreter's own allocations
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1:detect_odr_violation=0"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")],
                       capture_output=True, text=True, env=env, cwd=ROOT, timeout=900)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert " passed" in out
