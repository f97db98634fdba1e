"""Compile oracle/oracle.c into oracle/liboracle.so with the host C compiler.

Plain -O2: no -ffast-math, no vectorisation flags that could reassociate the
fp64 sums.  Test infrastructure only.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
OUT = os.path.join(HERE, "liboracle.so")


def build(cc: str | None = None, extra: list[str] | None = None, out: str = OUT) -> str:
    cc = cc or os.environ.get("CC", "gcc")
    cmd = [cc, "-std=c11", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fPIC",
           "-shared", "-Wall", "-Wextra", "-o", out + ".tmp", SRC, "-lm", "-lpthread"]
    if extra:
        cmd[1:1] = extra
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(extra=sys.argv[1:] or None))
