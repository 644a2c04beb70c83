"""Compile the fp64 CPU oracle (orc.c) into oracle/liborc.so with gcc.

Test infrastructure: the oracle is the checker of the HIP library, never part of
it.  ``build(extra_flags, out)`` also serves the mutation tests, which compile
deliberately wrong copies of the oracle into a temporary directory.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "orc.c")
LIB = os.path.join(HERE, "liborc.so")


def build(extra_flags=(), out=LIB, src=SRC):
    cmd = ["gcc", "-std=c99", "-O2", "-fPIC", "-shared", "-Wall", "-Wextra", "-Werror",
           "-D_POSIX_C_SOURCE=200809L", *extra_flags, src, "-o", out + ".tmp", "-lm", "-lpthread"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(sys.argv[1:]))
