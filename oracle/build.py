"""Build the fp64 CPU oracle (test infrastructure) with the host C compiler.

The oracle is plain C11 compiled without fast-math, so every fp64 operation rounds
as IEEE 754 prescribes.  Run as a script or through build_oracle().
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


def build_oracle(src=SRC, out=LIB, extra_flags=()):
    cc = os.environ.get("CC", "gcc")
    cmd = [cc, "-std=c11", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fPIC",
           "-shared", "-pthread", *extra_flags, src, "-o", out, "-lm"]
    subprocess.run(cmd, check=True)
    return out


if __name__ == "__main__":
    print(build_oracle(*sys.argv[1:2]))
