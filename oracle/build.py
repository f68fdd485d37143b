"""Build the CPU oracle library (liboracle.so) with g++.

Test infrastructure only: the oracle is a checker, never part of the product
path. It is compiled with plain IEEE double semantics: no -ffast-math, no
FMA contraction, no host-specific ISA flags.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False, src: str = None, out: str = None) -> str:
    src = src or os.path.join(HERE, "oracle.cpp")
    out = out or LIB
    cmd = [
        "g++", "-O3", "-std=c++17", "-fPIC", "-shared", "-pthread",
        "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra",
        "-I", HERE, src, "-o", out + ".tmp",
    ]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
