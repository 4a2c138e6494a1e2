"""Compile the CPU oracle (the Q4_K matmul and the KV-cache convert) into
oracle/liboracle_q4k.so (test infrastructure).

Plain gcc, -O2 with OpenMP, IEEE semantics kept: no -ffast-math, and no
floating-point contraction so every expression rounds as written.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRCS = [os.path.join(HERE, "q4k_oracle.c"), os.path.join(HERE, "kv_oracle.c")]
LIB = os.path.join(HERE, "liboracle_q4k.so")


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
           "-std=c11", "-Wall", "-Wextra", "-fPIC", "-shared",
           *SRCS, "-o", LIB + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
