"""Compile the CPU oracle into oracle/libbitnet_oracle.so with the host compiler.

TEST INFRASTRUCTURE ONLY: the oracle is the checker of the HIP library, never
part of it.  Plain C++17, no fast-math, no floating-point contraction, OpenMP
only to spread independent output rows over host threads.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "bitnet_oracle.cpp")
LIB = os.path.join(HERE, "libbitnet_oracle.so")

CXX_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-shared", "-fopenmp",
             "-fno-fast-math", "-ffp-contract=off", "-Wall", "-Wextra"]


def build(src=SRC, out=LIB, extra_flags=()):
    """Compile `src` to the shared library `out`; returns the output path."""
    cxx = os.environ.get("CXX", "g++")
    tmp = out + ".tmp"
    cmd = [cxx, *CXX_FLAGS, *extra_flags, src, "-o", tmp]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build())
