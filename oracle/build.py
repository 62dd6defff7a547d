"""Build the CPU oracle shared library (test infrastructure only) from
nvfp4_oracle.c and mxfp4_oracle.c.

Plain C11, -O2, -ffp-contract=off so that every fp32 operation in the block
quantization is rounded on its own, as the oracle's arithmetic assumes.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRCS = [os.path.join(HERE, "nvfp4_oracle.c"), os.path.join(HERE, "mxfp4_oracle.c")]
LIB = os.path.join(HERE, "liborc.so")


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math", "-Wall",
           "-Wextra", "-fPIC", "-shared", "-pthread", "-o", tmp] + SRCS + ["-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
