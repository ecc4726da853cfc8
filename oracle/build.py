"""Build step for the fp64 oracle library (test infrastructure; plain gcc, no HIP)."""
from __future__ import annotations

import os
import subprocess

_HERE = os.path.dirname(os.path.abspath(__file__))


def oracle_lib_path() -> str:
    return os.path.join(_HERE, "libkda_oracle.so")


def build_oracle(verbose: bool = False) -> str:
    """Compile kda_oracle.c with gcc -O2 (no fast-math) and OpenMP into oracle/libkda_oracle.so."""
    src = os.path.join(_HERE, "kda_oracle.c")
    out = oracle_lib_path()
    tmp = out + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
           "-o", tmp, src, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build_oracle(verbose=True))
