"""Build the CPU oracle library (plain C++17, host only).

TEST INFRASTRUCTURE: the oracle is built so the tests, the smoke check and the
benchmark's CPU-baseline leg can load it; the product path never does.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libpa_oracle.so")
SRC = os.path.join(HERE, "pa_oracle.cpp")


def build(verbose: bool = False) -> str:
    cmd = [
        "g++", "-O2", "-std=c++17", "-ffp-contract=off", "-fno-fast-math",
        "-fPIC", "-shared", "-pthread", "-Wall", "-Wextra",
        SRC, "-o", LIB + ".tmp",
    ]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
