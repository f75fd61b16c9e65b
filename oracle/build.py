"""Build step for the CPU oracle (test infrastructure).

Compiles ``mxfp4_oracle.c`` with gcc into ``liboracle_mxfp4.so`` next to it.
Strict IEEE settings: no fast-math and no floating-point contraction, so every
rounding in the oracle is the one written in its source.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "mxfp4_oracle.c")
LIB = os.path.join(HERE, "liboracle_mxfp4.so")


def build(verbose: bool = False) -> str:
    cmd = [
        "gcc", "-O2", "-std=c11", "-fPIC", "-shared",
        "-ffp-contract=off", "-fno-fast-math", "-frounding-math",
        "-Wall", "-Wextra", "-Wno-unused-parameter",
        SRC, "-o", LIB + ".tmp", "-lm",
    ]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
