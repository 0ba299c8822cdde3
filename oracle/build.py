"""Build the fp64 CPU oracle (plain C, gcc + OpenMP) into a shared library.

Test infrastructure only: the product library never loads what this builds.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(HERE, "kda_oracle.c")
LIBRARY = os.path.join(HERE, "libkda_oracle.so")


SANITIZED = os.path.join(HERE, "libkda_oracle_san.so")
# Host AddressSanitizer + UndefinedBehaviorSanitizer build: every report is
# fatal.  A process that loads it must preload libasan (the interpreter itself
# is not instrumented).
SANITIZE_FLAGS = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                  "-fno-sanitize-recover=all"]


def build(source: str = SOURCE, output: str | None = None, quiet: bool = True,
          sanitize: bool = False) -> str:
    """Compile `source` with gcc into `output` (the plain or the sanitized
    library by default); returns the library path."""
    if output is None:
        output = SANITIZED if sanitize else LIBRARY
    opt = SANITIZE_FLAGS if sanitize else ["-O2"]
    cmd = ["gcc", *opt, "-std=c99", "-fopenmp", "-fPIC", "-shared",
           "-Wall", "-Werror", source, "-o", output + ".tmp", "-lm"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("oracle build failed:\n" + " ".join(cmd) + "\n" + res.stderr)
    os.replace(output + ".tmp", output)
    if not quiet:
        print("built", output)
    return output


if __name__ == "__main__":
    build(quiet=False)
    sys.exit(0)
