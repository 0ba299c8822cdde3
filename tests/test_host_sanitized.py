"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only): kda_api.hip -- every entry point's argument checks -- compiled
with host sanitizers and linked with the regular objects, then the ABI and
binding checks run against it in a child process with clang's ASan runtime
preloaded and every report fatal.  No call reaches a kernel."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_checks_under_asan_and_ubsan():
    from gated_delta_rule_42_amd import build as kbuild
    lib = kbuild.build_host_sanitized()
    env = dict(os.environ, LD_PRELOAD=kbuild.asan_runtime(), KDA_LIBRARY=lib,
               # The interpreter's and torch's own allocations are not the library's.
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:detect_odr_violation=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    # -s: a report goes to fd 2, which pytest would otherwise capture and lose
    # when the process aborts.
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-s", "-p", "no:cacheprovider",
                          os.path.join(ROOT, "tests", "test_abi.py"),
                          os.path.join(ROOT, "tests", "test_binding_checks.py")],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = res.stdout + res.stderr
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert res.returncode == 0, out[-4000:]
    assert " passed" in out
