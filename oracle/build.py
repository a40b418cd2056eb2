"""Compile the CPU oracle (moe_oracle.c) into liboracle.so with gcc.

Test infrastructure: building the checker is not using it; only the tests,
the smoke check and the benchmark's CPU-baseline leg load the result.
-ffp-contract=off keeps every fp32 multiply and add separately rounded, as the
oracle documents; -mavx2 only widens the vector registers gcc may use for the
16 independent partial sums (no change to any result).
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))


def build(verbose: bool = False) -> str:
    src = os.path.join(HERE, "moe_oracle.c")
    out = os.path.join(HERE, "liboracle.so")
    cmd = ["gcc", "-O3", "-mavx2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared", "-std=c11",
           "-Wall", "-Wextra", src, "-o", out + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
