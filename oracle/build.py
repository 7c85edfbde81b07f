"""Builds the CPU oracle (test infrastructure) into oracle/liboracle_topk.so.

Only the test suite, the package smoke check and the benchmark's CPU-baseline
leg load the result. Plain g++, -O3, no fast-math, C++17 threads.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle_topk.cpp")
LIB = os.path.join(HERE, "liboracle_topk.so")


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = ["g++", "-O3", "-std=c++17", "-shared", "-fPIC", "-pthread", SRC, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
