"""Build step for the CPU oracle (gcc, fp64, strict IEEE: no fast-math, no FMA
contraction).  Test infrastructure only."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "gdn_oracle.c")
LIB_PATH = os.path.join(HERE, "libgdn_oracle.so")


def build(verbose: bool = False) -> str:
    """Compile gdn_oracle.c into oracle/libgdn_oracle.so and return its path."""
    tmp = LIB_PATH + ".tmp"
    cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-pthread",
           "-ffp-contract=off", "-fno-fast-math", SRC, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
