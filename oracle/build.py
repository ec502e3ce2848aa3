"""Build oracle/liboracle.so from attn_oracle.c with gcc (fp64, OpenMP).

Test infrastructure only: the oracle is the independent CPU check of the HIP
attention library and shares nothing with it.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "attn_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


def build(src=SRC, out=LIB, extra_flags=(), quiet=False):
    """Compile the oracle C source into a shared library and return its path.

    -ffp-contract=off keeps every product and sum a separately rounded fp64
    operation, in the order the source states it.
    """
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
           *extra_flags, src, "-o", tmp, "-lm"]
    if not quiet:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    build(quiet="-q" in sys.argv)
