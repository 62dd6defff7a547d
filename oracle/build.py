"""Build the CPU oracle shared library (test infrastructure only) from
nvfp4_oracle.c and mxfp4_oracle.c.

Plain C11, -O2, -ffp-contract=off so that every fp32 operation in the block
quantization is rounded on its own, as the oracle's arithmetic assumes.

build(sanitize=True) builds the same sources with AddressSanitizer and
UndefinedBehaviorSanitizer (a host-only gcc build; no GPU code is involved),
for a test that runs the pins against it in a child process.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRCS = [os.path.join(HERE, "nvfp4_oracle.c"), os.path.join(HERE, "mxfp4_oracle.c")]
LIB = os.path.join(HERE, "liborc.so")
SANITIZE = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g"]


def build(verbose: bool = False, sanitize: bool = False, out: str = None) -> str:
    lib = out or (os.path.join(HERE, "liborc_san.so") if sanitize else LIB)
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math", "-Wall",
           "-Wextra", "-fPIC", "-shared", "-pthread"] + (SANITIZE if sanitize else []) + \
          ["-o", tmp] + SRCS + ["-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, lib)
    return lib


def sanitizer_runtime() -> str:
    """Path of gcc's AddressSanitizer runtime (it must be loaded first into a
    process that loads the sanitized library)."""
    r = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True, check=True)
    return r.stdout.strip()


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, sanitize="--sanitize" in sys.argv))
