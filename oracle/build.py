"""Build the CPU oracle library (test infrastructure; see oracle/__init__.py).

Plain g++ with no fast-math and no floating-point contraction, so the fp64
sums are evaluated exactly in the order the source writes them.
"""

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "lora_oracle.cpp")
LIB = os.path.join(HERE, "liblora_oracle.so")


def build(verbose: bool = False) -> str:
    cmd = ["g++", "-O2", "-std=c++17", "-fPIC", "-shared", "-pthread", "-ffp-contract=off",
           "-fno-fast-math", "-Wall", "-Wextra", SRC, "-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
