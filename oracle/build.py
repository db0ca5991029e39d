"""Build the CPU oracle (test infrastructure only) with the host C compiler.

Only the tests, the smoke check and the benchmark's CPU-baseline leg load the
result.  The product's HIP library is built separately and never links it.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "pa_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


def build(force: bool = True) -> str:
    """Compile pa_oracle.c into oracle/liboracle.so and return its path.

    Plain -O2 (no fast-math, no FMA contraction) so the double arithmetic is
    the IEEE arithmetic written in the source.
    """
    if not force and os.path.exists(LIB) and os.path.getmtime(LIB) >= os.path.getmtime(SRC):
        return LIB
    tmp = LIB + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared",
           "-Wall", "-Wextra", "-Werror", SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
