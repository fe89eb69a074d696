"""Compile the CPU oracle (plain C, gcc) into ``oracle/libsvref.so``.

Test infrastructure: the product library never links or loads it.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libsvref.so")


def build(verbose: bool = False) -> str:
    cmd = [
        "gcc", "-std=c11", "-O2", "-g", "-fPIC", "-shared",
        "-fno-fast-math", "-ffp-contract=off", "-Wall", "-Wextra",
        "-o", LIB + ".tmp", os.path.join(HERE, "svref.c"), "-lm",
    ]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
