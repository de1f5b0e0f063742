"""Compile the CPU oracle into oracle/libdsa_oracle.so with gcc.

Test infrastructure: plain C, -O2, OpenMP, no fast-math.  Run as a script or
call build().
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "dsa_oracle.c")
LIB = os.path.join(HERE, "libdsa_oracle.so")


def build(out=LIB, src=SRC, extra_flags=()):
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
           "-fno-fast-math", "-Wall", "-Wextra", "-o", out + ".tmp", src,
           "-lm", *extra_flags]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build())
