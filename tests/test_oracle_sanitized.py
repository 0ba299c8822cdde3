"""The C oracle under the host AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only): the oracle's pins and argument checks, run in a child process that
loads a -fsanitize=address,undefined build of oracle/kda_oracle.c, with every
sanitizer report fatal."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_oracle_pins_under_asan_and_ubsan():
    from oracle import build as obuild
    lib = obuild.build(sanitize=True)
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True,
                          check=True).stdout.strip()
    assert os.path.isabs(asan) and os.path.exists(asan), "libasan not found"
    env = dict(os.environ, LD_PRELOAD=asan, KDA_ORACLE_LIB=lib,
               # The interpreter's own allocations are not the oracle's leaks.
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    # -s: a sanitizer report goes to fd 2, which pytest would otherwise capture
    # and lose when the process aborts.
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-s", "-p", "no:cacheprovider",
                          os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = res.stdout + res.stderr
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert res.returncode == 0, out[-4000:]
    assert " passed" in out
