"""Compile the fp64 CPU oracle (test infrastructure) into oracle/liboracle.so with gcc."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "liboracle.so")


def build(src=None, out=None, extra=()):
    src = src or os.path.join(HERE, "oracle.c")
    out = out or LIB
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-Wall", "-Wextra", "-fno-fast-math", "-pthread",
           *extra, src, "-o", out, "-lm"]
    subprocess.run(cmd, check=True)
    return out


if __name__ == "__main__":
    print(build())
