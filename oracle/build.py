"""Compile the CPU oracle (plain C, single-threaded) into oracle/liboracle.so.

Test infrastructure: only the tests, the smoke check and the benchmark's CPU
baseline load the result.  No fast-math: every step must keep IEEE semantics.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "fp4q_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-O2", "-std=c99", "-Wall", "-Wextra", "-fPIC", "-shared",
           "-fno-fast-math", "-ffp-contract=off", "-o", LIB + ".tmp", SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
