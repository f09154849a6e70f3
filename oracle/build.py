"""Build the CPU oracle library (``oracle/liboracle.so``) with plain gcc.

TEST INFRASTRUCTURE: the oracle is built so that tests, the smoke check and
the benchmark's CPU-baseline leg can check the HIP path; the product library
never loads it.

Flags: ``-O2 -fopenmp -ffp-contract=off`` and no fast-math, so every double
product and sum is rounded exactly as written in ``oracle.c``.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

CFLAGS = ["-std=c11", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
          "-Wall", "-Wextra", "-shared", "-fPIC"]


def build(src: str = SRC, out: str = LIB, extra: list[str] | None = None) -> str:
    """Compile ``src`` into the shared library ``out`` and return its path."""
    cmd = ["gcc", *CFLAGS, *(extra or []), "-I", HERE, src, "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(extra=sys.argv[1:]))
