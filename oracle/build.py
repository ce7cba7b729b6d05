"""Build the CPU oracle (test infrastructure) with gcc.

    python oracle/build.py            -> oracle/liboracle.so
    build(mutation=True)              -> a copy with the planted int32-offset
                                         mistake, for the discrimination test
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "pa_oracle.c")


def build(out: str | None = None, mutation: bool = False, quiet: bool = True) -> str:
    out = out or os.path.join(HERE, "liboracle_mut.so" if mutation else "liboracle.so")
    cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-std=c11",
           "-Wall", "-Wextra", "-Wno-unused-parameter", "-shared", "-fPIC", SRC, "-o",
           out + ".tmp", "-lm"]
    if mutation:
        cmd.insert(1, "-DORACLE_MUTATION_INT32_BLOCK_OFFSET")
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("oracle build failed:\n" + res.stdout + res.stderr)
    if not quiet and res.stderr:
        print(res.stderr, file=sys.stderr)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(quiet=False))
