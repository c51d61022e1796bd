"""Build step for the fp64 CPU oracle (test infrastructure only).

Compiles ``attn_oracle.c`` with gcc into ``liboracle.so`` next to it.  Plain
``-O2``: no fast-math, so every floating-point operation is the IEEE fp64
operation the source spells out.

``build(sanitize=True)`` writes ``liboracle_san.so`` instead: the same source
under AddressSanitizer and UndefinedBehaviorSanitizer (any report aborts).  A
process that loads it needs gcc's ASan runtime preloaded (``asan_runtime()``);
with ``ORACLE_SANITIZE=1`` in the environment the oracle package loads that
build, and the mutant tests compile their copies with the same flags.
"""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "attn_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")
LIB_SAN = os.path.join(HERE, "liboracle_san.so")

SANITIZE_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                  "-fno-omit-frame-pointer", "-g"]


def sanitize_requested() -> bool:
    return os.environ.get("ORACLE_SANITIZE", "") == "1"


def cflags(sanitize: bool = False, opt: str = "-O2") -> list:
    """gcc flags of a shared oracle build (without the output and sources)."""
    flags = [opt, "-std=c11", "-fPIC", "-shared", "-fopenmp", "-Wall", "-Wextra"]
    return flags + (SANITIZE_FLAGS if sanitize else [])


def asan_runtime() -> str | None:
    """Path of gcc's ASan runtime (to preload into a Python process), or None."""
    out = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True)
    path = out.stdout.strip()
    return path if out.returncode == 0 and os.path.isabs(path) and os.path.exists(path) else None


def build(verbose: bool = False, sanitize: bool = False) -> str:
    lib = LIB_SAN if sanitize else LIB
    cmd = ["gcc"] + cflags(sanitize) + ["-o", lib + ".tmp", SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(lib + ".tmp", lib)
    return lib


if __name__ == "__main__":
    import sys
    print(build(verbose=True, sanitize="--sanitize" in sys.argv[1:]))
