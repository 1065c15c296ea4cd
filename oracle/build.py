"""Build the fp64 CPU oracle (test infrastructure) as oracle/liblinattn_oracle.so.

Plain gcc, OpenMP, no FMA contraction and no -march=native, so the library is
portable to whatever x86-64 host runs the tests and the arithmetic stays the
plain sequence of multiplies and adds written in the source.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "linattn_oracle.c")
LIB = os.path.join(HERE, "liblinattn_oracle.so")


SAN_LIB = os.path.join(HERE, "liblinattn_oracle_san.so")


def build(verbose: bool = False, sanitize: bool = False) -> str:
    """sanitize: an AddressSanitizer + UndefinedBehaviorSanitizer build into
    liblinattn_oracle_san.so (load it with SANA_ORACLE_LIB and libasan
    preloaded) for the host sanitizer pass over the oracle's tests."""
    lib = SAN_LIB if sanitize else LIB
    tmp = lib + ".tmp"
    san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g"] \
        if sanitize else []
    cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
           "-Wall", "-Wextra", "-Werror", *san, SRC, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, sanitize="--sanitize" in sys.argv))
