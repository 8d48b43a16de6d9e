"""Builds the CPU oracle (plain C, OpenMP) into ``oracle/liboracle.so``.

Test infrastructure only: the tests compare the HIP path with it; it is never part of the product.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")
SAN_LIB = os.path.join(HERE, "liboracle_san.so")  # AddressSanitizer + UndefinedBehaviorSanitizer build
SAN_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g"]


def build(verbose: bool = False, sanitize: bool = False) -> str:
    """Builds the oracle library (``sanitize``: the ASan/UBSan build, loaded
    by the CPU tests when ``ORACLE_LIB`` names it and the ASan runtime is
    preloaded; a UBSan finding aborts)."""
    out = SAN_LIB if sanitize else LIB
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O1" if sanitize else "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-mf16c",
           "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra", *(SAN_FLAGS if sanitize else []),
           SRC, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True, sanitize="--sanitize" in sys.argv))
